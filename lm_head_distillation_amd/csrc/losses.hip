// Two standalone losses over given distributions, one pass each (every
// element's loss and gradient depend on that element alone; rows reduce their
// loss through the same slice partials as the logit-space JSD):
//
//  * Generalized JSD in log-probability space (Liger-Kernel PR #1352, Open
//    question 3: the public JSD op takes log-probabilities). Inputs x = ln Q
//    (student) and y = ln P (teacher), taken as given, D = y - x:
//      forward KL (beta 0): l = P D,           g = -P
//      reverse KL (beta 1): l = -Q D,          g = Q - Q D
//      generalized:          r = ln(beta e^D + 1 - beta),
//                            l = beta P (D - r) - (1-beta) Q r,  g = -(1-beta) Q r
//    with g = dl/dx, elementwise (no softmax chain rule: the inputs are the
//    variables). r and D - r come from mix_log for fp32 inputs, as in the
//    logit path, and from jsd_r_direct for bf16 inputs, whose own rounding
//    (2^-9 |x|) outweighs the difference. An exact tie P == Q gives l = 0 and, in the generalized branch,
//    g = 0 (PR #1374); zero-probability factors contribute 0 (0 log 0 = 0).
//
//  * Total variation distance (PR #1374 "Fix TVD gradient at p == q"):
//    l = |p - q| / 2, dl/dp = +1/2 (p > q), -1/2 (p < q), 0 (p == q).
#include "elem_math.h"
#include "kernels.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fljsd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.44269504088896341f;

template <int MODE, bool DIRECT>
__device__ inline void logprob_terms(float x, float y, float beta, const BetaWeights& bw, float& l,
                                     float& g) {
  const float Q = hw_exp2(x * kLog2e);
  const float P = hw_exp2(y * kLog2e);
  if (P == Q) {  // exact tie (also both zero): D = 0
    l = 0.f;
    g = MODE == kModeForwardKL ? -P : (MODE == kModeReverseKL ? Q : 0.f);
    return;
  }
  const float D = y - x;
  if (MODE == kModeForwardKL) {
    l = P > 0.f ? P * D : 0.f;
    g = -P;
  } else if (MODE == kModeReverseKL) {
    const float qd = Q > 0.f ? Q * D : 0.f;
    l = -qd;
    g = Q - qd;
  } else {
    float r, dmr;
    if constexpr (DIRECT) {
      jsd_r_direct(D, D * kLog2e, beta, r, dmr);
    } else {
      r = mix_log(D, D * kLog2e, bw.r);
      dmr = -mix_log(-D, -D * kLog2e, bw.dmr);
    }
    const float tp = P > 0.f ? beta * P * dmr : 0.f;
    const float tq = Q > 0.f ? (1.f - beta) * Q * r : 0.f;
    l = tp - tq;
    g = -tq;
  }
}

// Block sum of one float per thread; thread 0 gets the total.
__device__ inline float block_sum(float x) {
  x = wave_sum(x);
  __shared__ float sh[kWaves];
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) sh[wave] = x;
  __syncthreads();
  float acc = sh[0];
  for (int w = 1; w < kWaves; ++w) acc += sh[w];
  return acc;
}

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void logprob_jsd_kernel(ElemArgs a) {
  const int64_t row = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_w;
  const int64_t v1 = min(a.V, v0 + a.slice_w);
  const T* xs = static_cast<const T*>(a.a) + row * a.ld;
  const T* ys = static_cast<const T*>(a.b) + row * a.ld;
  T* gr = a.grad ? static_cast<T*>(a.grad) + row * a.ld : nullptr;
  const BetaWeights bw = beta_weights(a.beta);
  float lsum = 0.f;
  for (int64_t v = v0 + threadIdx.x * 8; v < v1; v += kThreads * 8) {
    const int n = static_cast<int>(min<int64_t>(8, v1 - v));
    float x[8], y[8], out[8];
    load8(xs, v, n, a.vec_ok, x);
    load8(ys, v, n, a.vec_ok, y);
    // Columns past the row end load as -inf in both rows (Q = P = 0): an
    // exact tie, whose loss term is exactly 0.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float l, g;
      logprob_terms<MODE, sizeof(T) == 2>(x[i], y[i], a.beta, bw, l, g);
      lsum += l;
      out[i] = g * a.grad_scale;
    }
    if (gr) store8(gr, v, n, a.vec_ok, out);
  }
  const float tot = block_sum(lsum);
  if (threadIdx.x == 0) a.lg[row * a.S + s] = make_float2(tot, 0.f);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void tvd_kernel(ElemArgs a) {
  const int64_t row = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_w;
  const int64_t v1 = min(a.V, v0 + a.slice_w);
  const T* ps = static_cast<const T*>(a.a) + row * a.ld;
  const T* qs = static_cast<const T*>(a.b) + row * a.ld;
  T* gr = a.grad ? static_cast<T*>(a.grad) + row * a.ld : nullptr;
  float* el = a.elem_loss ? a.elem_loss + row * a.V : nullptr;
  const bool el_vec = (a.V & 3) == 0;
  const float half = 0.5f * a.grad_scale;
  float lsum = 0.f;
  for (int64_t v = v0 + threadIdx.x * 8; v < v1; v += kThreads * 8) {
    const int n = static_cast<int>(min<int64_t>(8, v1 - v));
    float p[8], q[8], out[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) l[i] = 0.f;
    load8(ps, v, n, a.vec_ok, p, 0.f);
    load8(qs, v, n, a.vec_ok, q, 0.f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float d = p[i] - q[i];
      l[i] = 0.5f * fabsf(d);
      lsum += l[i];   // masked lanes load 0 for both
      out[i] = d > 0.f ? half : (d < 0.f ? -half : 0.f);
    }
    if (gr) store8(gr, v, n, a.vec_ok, out);
    if (el) store8(el, v, n, el_vec, l);
  }
  const float tot = block_sum(lsum);
  if (threadIdx.x == 0) a.lg[row * a.S + s] = make_float2(tot, 0.f);
}

template <typename T>
hipError_t launch_logprob_t(const ElemArgs& a, hipStream_t s, dim3 grid) {
  const dim3 block(kThreads);
  if (a.mode == kModeForwardKL)
    hipLaunchKernelGGL((logprob_jsd_kernel<T, kModeForwardKL>), grid, block, 0, s, a);
  else if (a.mode == kModeReverseKL)
    hipLaunchKernelGGL((logprob_jsd_kernel<T, kModeReverseKL>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((logprob_jsd_kernel<T, kModeGeneralized>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_logprob_jsd(const ElemArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.rows), static_cast<unsigned>(a.S));
  return dtype == 0 ? launch_logprob_t<float>(a, s, grid) : launch_logprob_t<uint16_t>(a, s, grid);
}

hipError_t launch_tvd(const ElemArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.rows), static_cast<unsigned>(a.S));
  if (dtype == 0)
    hipLaunchKernelGGL(tvd_kernel<float>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(tvd_kernel<uint16_t>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fljsd
