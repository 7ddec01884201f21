// Online-softmax generalized JSD over logits rows, in three passes
// (Liger-Kernel PR #1352 "Fuse log-softmax into fused_linear_jsd kernel",
// Details):
//   pass 1  row statistics m and d (running max and denominator, Milakov &
//           Gimelshein's online normalizer) for student and teacher together;
//   pass 2  the per-row loss and the cross-column term dX_sum;
//   pass 3  dX, written over the student logits when the caller asks for it
//           in place.
// Everything from the loaded logit onward is fp32 (PR #1352 Details: the cast
// happens at load). Exponentials are base 2: logits are pre-scaled by
// log2(e)/T so the hardware exp2 path evaluates e^x (PR #1352 Details, last
// bullet). A row may be split into S slices, each a workgroup; the slices'
// partial statistics and sums are merged in a fixed order, so results are
// deterministic run to run.
//
// Per element, with a = log2 of a probability (a_s = y_s - L_s, a_t = y_t -
// L_t, y = z log2(e)/T, L = m + log2 d), Q = 2^a_s (student), P = 2^a_t
// (teacher) and D = ln P - ln Q = (a_t - a_s) ln 2:
//   generalized: r = ln(beta e^D + 1 - beta), evaluated as
//                  D <  0: log1p(beta expm1(D))
//                  D >= 0: D + log1p((1-beta) expm1(-D))
//                ln(P/M) = D - r, ln(Q/M) = -r,
//                l = beta P (D - r) - (1-beta) Q r,   g = -(1-beta) Q r,
//                dA = g - Q G with G = sum_v g (dX_sum)
//   forward KL:  l = P D - P + Q,  dA = Q - P          (sum_v P = 1 exactly)
//   reverse KL:  l = P - Q - Q D,  G = sum_v l,  dA = -Q D - Q G
// and an exact tie P == Q gives l = g = 0 (PR #1374 "Fix TVD gradient at
// p == q": one predicate and one select per element).
// The KL terms carry "- P + Q" (which sums to zero over a row) so that each
// term is O(D^2) and non-negative: the plain P D terms are O(D) and cancel
// across the row, which turns the fp32 rounding of the row normalizers into a
// first-order error of the loss. Near D = 0 the terms come from their Taylor
// series; the generalized divergence needs no such care (its derivative with
// respect to a normalizer error is itself O(loss)).
// y = z log2(e)/T is rounded once (no fused multiply-add) so every pass sees
// the same y; the row maximum then gives a = y - L exactly where d = 1.
#include "kernels.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

namespace fljsd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLn2 = 0.693147180559945309f;

__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ inline uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);                       // round to nearest even
  return u >> 16;
}

// Load up to 8 consecutive elements starting at column v; lanes at or past n
// read as -inf (a masked column carries no probability mass). A full group
// uses 16-byte loads when `vec` says the rows are 16-byte aligned.
__device__ inline void load8(const float* p, int64_t v, int n, bool vec, float* x) {
  if (n == 8 && vec) {
    const float4 a = *reinterpret_cast<const float4*>(p + v);
    const float4 b = *reinterpret_cast<const float4*>(p + v + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = i < n ? p[v + i] : -INFINITY;
  }
}

__device__ inline void load8(const uint16_t* p, int64_t v, int n, bool vec, float* x) {
  if (n == 8 && vec) {
    const uint4 q = *reinterpret_cast<const uint4*>(p + v);
    x[0] = bf16_lo(q.x); x[1] = bf16_hi(q.x);
    x[2] = bf16_lo(q.y); x[3] = bf16_hi(q.y);
    x[4] = bf16_lo(q.z); x[5] = bf16_hi(q.z);
    x[6] = bf16_lo(q.w); x[7] = bf16_hi(q.w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = i < n ? __uint_as_float(uint32_t(p[v + i]) << 16) : -INFINITY;
  }
}

__device__ inline void store8(float* p, int64_t v, int n, bool vec, const float* x) {
  if (n == 8 && vec) {
    *reinterpret_cast<float4*>(p + v) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + v + 4) = make_float4(x[4], x[5], x[6], x[7]);
  } else {
    for (int i = 0; i < n; ++i) p[v + i] = x[i];
  }
}

__device__ inline void store8(uint16_t* p, int64_t v, int n, bool vec, const float* x) {
  if (n == 8 && vec) {
    uint4 q;
    q.x = f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16);
    q.y = f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16);
    q.z = f32_to_bf16_bits(x[4]) | (f32_to_bf16_bits(x[5]) << 16);
    q.w = f32_to_bf16_bits(x[6]) | (f32_to_bf16_bits(x[7]) << 16);
    *reinterpret_cast<uint4*>(p + v) = q;
  } else {
    for (int i = 0; i < n; ++i) p[v + i] = static_cast<uint16_t>(f32_to_bf16_bits(x[i]));
  }
}

// y = z * log2(e)/T, rounded to fp32 on its own: contraction into a later
// subtraction is switched off so every pass computes bit-identical y.
__device__ inline float scaled_logit(float z, float k2) {
#pragma clang fp contract(off)
  return z * k2;
}

// Merge of two (max, denominator) pairs in base 2. Commutative bit for bit
// (max and a two-term IEEE sum are), so both butterfly partners agree.
__device__ inline void md_merge(float& m, float& d, float mo, float dof) {
  const float M = fmaxf(m, mo);
  if (M == -INFINITY) {
    m = -INFINITY;
    d = 0.f;
    return;
  }
  d = d * exp2f(m - M) + dof * exp2f(mo - M);
  m = M;
}

// Fold 8 scaled logits into a running (max, denominator).
__device__ inline void md_update8(float& m, float& d, const float* y) {
  float mx = y[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, y[i]);
  if (mx == -INFINITY) return;
  if (mx > m) {
    d *= exp2f(m - mx);
    m = mx;
  }
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += exp2f(y[i] - m);
  d += acc;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ inline void wave_md(float& m, float& d) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float mo = __shfl_xor(m, o, 64);
    const float dof = __shfl_xor(d, o, 64);
    md_merge(m, d, mo, dof);
  }
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

// Per-element terms of the divergence; see the file comment. Outputs: the
// probabilities Q and P, the loss term l, the gradient term g (dA = g - Q G)
// and gacc, the term summed into G.
template <int MODE>
__device__ inline void jsd_terms(float as, float at, float beta, float& Q, float& P, float& l,
                                 float& g, float& gacc) {
  Q = exp2f(as);
  P = exp2f(at);
  if (P == Q) {  // exact tie: no loss, no gradient term
    l = 0.f;
    g = 0.f;
    gacc = 0.f;
    return;
  }
  const float D = (at - as) * kLn2;
  if (MODE == kModeForwardKL) {
    l = fabsf(D) < 0.25f ? Q * kl_fwd_series(D) : P * D - (P - Q);
    g = -P;
    gacc = 0.f;  // dA = Q - P needs no row sum
  } else if (MODE == kModeReverseKL) {
    l = fabsf(D) < 0.25f ? Q * kl_rev_series(D) : (P - Q) - Q * D;
    g = -Q * D;
    gacc = l;    // G = KL(Q||P), the row loss
  } else {
    float r, dmr;
    if (D >= 0.f) {
      const float u = log1pf((1.f - beta) * expm1f(-D));
      r = D + u;
      dmr = -u;
    } else {
      r = log1pf(beta * expm1f(D));
      dmr = D - r;
    }
    l = beta * P * dmr - (1.f - beta) * Q * r;
    g = -(1.f - beta) * Q * r;
    gacc = g;
  }
}

// Row statistics from the S pass-1 partials, merged in slice order by one
// thread and broadcast through LDS. Returns L_s = m_s + log2 d_s and L_t.
__device__ inline void row_log_norms(const JsdArgs& a, int64_t row, float& Ls, float& Lt) {
  __shared__ float2 sh_L;
  if (threadIdx.x == 0) {
    const float4* st = a.stats + row * a.S;
    float4 acc = st[0];
    for (int s = 1; s < a.S; ++s) {
      const float4 o = st[s];
      md_merge(acc.x, acc.y, o.x, o.y);
      md_merge(acc.z, acc.w, o.z, o.w);
    }
    sh_L = make_float2(acc.x + log2f(acc.y), acc.z + log2f(acc.w));
  }
  __syncthreads();
  Ls = sh_L.x;
  Lt = sh_L.y;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void jsd_stats_kernel(JsdArgs a) {
  const int64_t row = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_w;
  const int64_t v1 = min(a.V, v0 + a.slice_w);
  const T* zs = static_cast<const T*>(a.zs) + row * a.ld;
  const T* zt = static_cast<const T*>(a.zt) + row * a.ld;
  float ms = -INFINITY, ds = 0.f, mt = -INFINITY, dt = 0.f;
  for (int64_t v = v0 + threadIdx.x * 8; v < v1; v += kThreads * 8) {
    const int n = static_cast<int>(min<int64_t>(8, v1 - v));
    float ys[8], yt[8];
    load8(zs, v, n, a.vec_ok, ys);
    load8(zt, v, n, a.vec_ok, yt);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ys[i] = scaled_logit(ys[i], a.k2);
      yt[i] = scaled_logit(yt[i], a.k2);
    }
    md_update8(ms, ds, ys);
    md_update8(mt, dt, yt);
  }
  wave_md(ms, ds);
  wave_md(mt, dt);
  __shared__ float4 sh[kWaves];
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) sh[wave] = make_float4(ms, ds, mt, dt);
  __syncthreads();
  if (threadIdx.x == 0) {
    float4 acc = sh[0];
    for (int w = 1; w < kWaves; ++w) {
      md_merge(acc.x, acc.y, sh[w].x, sh[w].y);
      md_merge(acc.z, acc.w, sh[w].z, sh[w].w);
    }
    a.stats[row * a.S + s] = acc;
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
  float Ls, Lt;
  row_log_norms(a, row, Ls, Lt);
  float lsum = 0.f, gsum = 0.f;
  for (int64_t v = v0 + threadIdx.x * 8; v < v1; v += kThreads * 8) {
    const int n = static_cast<int>(min<int64_t>(8, v1 - v));
    float ys[8], yt[8];
    load8(zs, v, n, a.vec_ok, ys);
    load8(zt, v, n, a.vec_ok, yt);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < n) {
        float Q, P, l, g, gacc;
        jsd_terms<MODE>(scaled_logit(ys[i], a.k2) - Ls, scaled_logit(yt[i], a.k2) - Lt, a.beta, Q, P,
                        l, g, gacc);
        lsum += l;
        gsum += gacc;
      }
    }
  }
  lsum = wave_sum(lsum);
  gsum = wave_sum(gsum);
  __shared__ float2 sh[kWaves];
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) sh[wave] = make_float2(lsum, gsum);
  __syncthreads();
  if (threadIdx.x == 0) {
    float2 acc = sh[0];
    for (int w = 1; w < kWaves; ++w) {
      acc.x += sh[w].x;
      acc.y += sh[w].y;
    }
    a.lg[row * a.S + s] = acc;
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
  float Ls, Lt;
  row_log_norms(a, row, Ls, Lt);
  __shared__ float sh_G;
  if (threadIdx.x == 0) {
    const float2* lg = a.lg + row * a.S;
    float2 acc = lg[0];
    for (int k = 1; k < a.S; ++k) {
      acc.x += lg[k].x;
      acc.y += lg[k].y;
    }
    sh_G = acc.y;
    if (s == 0) a.row_loss[row] = acc.x;
  }
  __syncthreads();
  const float G = sh_G;
  for (int64_t v = v0 + threadIdx.x * 8; v < v1; v += kThreads * 8) {
    const int n = static_cast<int>(min<int64_t>(8, v1 - v));
    float ys[8], yt[8], out[8];
    load8(zs, v, n, a.vec_ok, ys);
    load8(zt, v, n, a.vec_ok, yt);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float Q, P, l, g, gacc;
      jsd_terms<MODE>(scaled_logit(ys[i], a.k2) - Ls, scaled_logit(yt[i], a.k2) - Lt, a.beta, Q, P, l,
                      g, gacc);
      const float dA = (MODE == kModeForwardKL) ? (Q - P) : (g - Q * G);
      out[i] = dA * a.grad_scale;
    }
    store8(gr, v, n, a.vec_ok, out);
  }
}

__global__ __launch_bounds__(64) void jsd_row_loss_kernel(JsdArgs a) {
  const int64_t row = blockIdx.x;
  if (threadIdx.x == 0) {
    const float2* lg = a.lg + row * a.S;
    float acc = lg[0].x;
    for (int k = 1; k < a.S; ++k) acc += lg[k].x;
    a.row_loss[row] = acc;
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
    float x[4] = {acc.x, acc.y, acc.z, acc.w};
    T* o = out + m * ldo + c;
    if constexpr (sizeof(T) == 4) {
      *reinterpret_cast<float4*>(o) = acc;
    } else {
      uint2 q;
      q.x = f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16);
      q.y = f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16);
      *reinterpret_cast<uint2*>(o) = q;
    }
  }
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
  const dim3 block(kThreads);
  if (dtype == 1) {
    if (a.mode == kModeForwardKL)
      hipLaunchKernelGGL((jsd_loss_kernel<uint16_t, kModeForwardKL>), grid, block, 0, s, a);
    else if (a.mode == kModeReverseKL)
      hipLaunchKernelGGL((jsd_loss_kernel<uint16_t, kModeReverseKL>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((jsd_loss_kernel<uint16_t, kModeGeneralized>), grid, block, 0, s, a);
  } else {
    if (a.mode == kModeForwardKL)
      hipLaunchKernelGGL((jsd_loss_kernel<float, kModeForwardKL>), grid, block, 0, s, a);
    else if (a.mode == kModeReverseKL)
      hipLaunchKernelGGL((jsd_loss_kernel<float, kModeReverseKL>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((jsd_loss_kernel<float, kModeGeneralized>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_jsd_grad(const JsdArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.rows), static_cast<unsigned>(a.S));
  const dim3 block(kThreads);
  if (dtype == 1) {
    if (a.mode == kModeForwardKL)
      hipLaunchKernelGGL((jsd_grad_kernel<uint16_t, kModeForwardKL>), grid, block, 0, s, a);
    else if (a.mode == kModeReverseKL)
      hipLaunchKernelGGL((jsd_grad_kernel<uint16_t, kModeReverseKL>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((jsd_grad_kernel<uint16_t, kModeGeneralized>), grid, block, 0, s, a);
  } else {
    if (a.mode == kModeForwardKL)
      hipLaunchKernelGGL((jsd_grad_kernel<float, kModeForwardKL>), grid, block, 0, s, a);
    else if (a.mode == kModeReverseKL)
      hipLaunchKernelGGL((jsd_grad_kernel<float, kModeReverseKL>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((jsd_grad_kernel<float, kModeGeneralized>), grid, block, 0, s, a);
  }
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
