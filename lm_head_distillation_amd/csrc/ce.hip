// Cross-entropy with hard labels over a chunk of lm_head logits: the
// fused-linear cross-entropy pattern that Liger-Kernel PR #1352 (Details)
// carries over to JSD, with CE's two passes (the online softmax of Milakov &
// Gimelshein for the row statistics, then the gradient written over the
// logits in place).
//
// Per row with label y and label smoothing eps, q = softmax(z):
//   loss = lse - (1 - eps) z_y - (eps / V) sum_v z_v,   lse = ln sum_v e^z_v
//   dz_v = scale (q_v - eps / V - (1 - eps) [v == y])
// A row whose label is the ignore index or lies outside [0, V) has loss 0
// and gradient 0. The scale comes from a count over all rows of the call
// (reduction mean divides by the number of counted rows), computed on the
// device before the first chunk, so chunking does not change it.
#include "elem_math.h"
#include "kernels.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace fljsd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.44269504088896341f;
constexpr int kScaleThreads = 1024;
// fljsd_reduction values (include/fljsd.h).
constexpr int kRedBatchmean = 0, kRedMean = 2;

__device__ inline bool counted(int64_t y, int64_t V, int64_t ignore_index) {
  return y != ignore_index && y >= 0 && y < V;
}

__global__ __launch_bounds__(kScaleThreads) void ce_scale_kernel(const int64_t* labels, int64_t BT,
                                                                 int64_t V, int64_t ignore_index,
                                                                 int reduction, float* scale) {
  int64_t n = 0;
  for (int64_t i = threadIdx.x; i < BT; i += kScaleThreads) n += counted(labels[i], V, ignore_index);
  __shared__ int64_t sh[kScaleThreads];
  sh[threadIdx.x] = n;
  __syncthreads();
  for (int w = kScaleThreads / 2; w >= 1; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int64_t cnt = sh[0];
    float g = 1.f, l = 1.f;
    if (reduction == kRedMean) {
      g = cnt > 0 ? static_cast<float>(1.0 / static_cast<double>(cnt)) : 0.f;
      l = cnt > 0 ? g : NAN;
    } else if (reduction == kRedBatchmean) {
      g = l = static_cast<float>(1.0 / static_cast<double>(BT));
    }
    scale[0] = g;
    scale[1] = l;
  }
}

template <typename T>
__device__ inline float load1(const T* p);
template <>
__device__ inline float load1<float>(const float* p) { return *p; }
template <>
__device__ inline float load1<uint16_t>(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void ce_stats_kernel(CeArgs a) {
  const int64_t row = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_w;
  const int64_t v1 = min(a.V, v0 + a.slice_w);
  const T* z = static_cast<const T*>(a.z) + row * a.ld;
  float m = -INFINITY, d = 0.f, sz = 0.f;
  for (int64_t v = v0 + threadIdx.x * 8; v < v1; v += kThreads * 8) {
    const int n = static_cast<int>(min<int64_t>(8, v1 - v));
    float x[8];
    load8(z, v, n, a.vec_ok, x);
    md_update8(m, d, x, kLog2e);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < n) sz += x[i];
  }
  wave_md(m, d, kLog2e);
  sz = wave_sum(sz);
  __shared__ float4 sh[kWaves];
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) sh[wave] = make_float4(m, d, sz, 0.f);
  __syncthreads();
  if (threadIdx.x == 0) {
    float4 acc = sh[0];
    for (int w = 1; w < kWaves; ++w) {
      md_merge(acc.x, acc.y, sh[w].x, sh[w].y, kLog2e);
      acc.z += sh[w].z;
    }
    a.stats[row * a.S + s] = acc;
    const int64_t y = a.labels[row];
    if (counted(y, a.V, a.ignore_index) && y >= v0 && y < v1) a.zy[row] = load1<T>(z + y);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void ce_grad_kernel(CeArgs a, bool write_grad) {
  const int64_t row = blockIdx.x;
  const int s = blockIdx.y;
  __shared__ float4 sh_st;   // (m, log2 d, sum z, -)
  const int64_t y = a.labels[row];
  const bool ok = counted(y, a.V, a.ignore_index);
  if (threadIdx.x == 0) {
    const float4* st = a.stats + row * a.S;
    float4 acc = st[0];
    for (int j = 1; j < a.S; ++j) {
      md_merge(acc.x, acc.y, st[j].x, st[j].y, kLog2e);
      acc.z += st[j].z;
    }
    sh_st = make_float4(acc.x, hw_log2(acc.y), acc.z, 0.f);
    if (s == 0) {
      const float lse = acc.x + sh_st.y * 0.693147180559945309f;
      const float V = static_cast<float>(a.V);
      a.row_loss[row] = ok ? lse - (1.f - a.eps) * a.zy[row] - (a.eps / V) * acc.z : 0.f;
    }
  }
  if (!write_grad) return;
  __syncthreads();
  const float m = sh_st.x, l2d = sh_st.y;
  const float gs = ok ? a.scale[0] : 0.f;
  const float off = a.eps / static_cast<float>(a.V);
  const float hit = 1.f - a.eps;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_w;
  const int64_t v1 = min(a.V, v0 + a.slice_w);
  const T* z = static_cast<const T*>(a.z) + row * a.ld;
  T* gr = static_cast<T*>(a.grad) + row * a.ld;
  for (int64_t v = v0 + threadIdx.x * 8; v < v1; v += kThreads * 8) {
    const int n = static_cast<int>(min<int64_t>(8, v1 - v));
    float x[8], out[8];
    load8(z, v, n, a.vec_ok, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = hw_exp2((x[i] - m) * kLog2e - l2d);
      const float dz = q - off - (v + i == y ? hit : 0.f);
      out[i] = ok ? dz * gs : 0.f;
    }
    store8(gr, v, n, a.vec_ok, out);
  }
}

constexpr int kReduceThreads = 1024;

__global__ __launch_bounds__(kReduceThreads) void loss_reduce_dev_kernel(const float* row_loss,
                                                                         int64_t n,
                                                                         const float* scale,
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
  if (threadIdx.x == 0) loss[0] = static_cast<float>(sh[0] * static_cast<double>(scale[1]));
}

}  // namespace

hipError_t launch_ce_scale(const int64_t* labels, int64_t BT, int64_t V, int64_t ignore_index,
                           int reduction, float* scale, hipStream_t s) {
  hipLaunchKernelGGL(ce_scale_kernel, dim3(1), dim3(kScaleThreads), 0, s, labels, BT, V,
                     ignore_index, reduction, scale);
  return hipGetLastError();
}

hipError_t launch_ce_stats(const CeArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.rows), static_cast<unsigned>(a.S));
  if (dtype == 0)
    hipLaunchKernelGGL(ce_stats_kernel<float>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(ce_stats_kernel<uint16_t>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ce_grad(const CeArgs& a, int dtype, bool write_grad, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.rows), static_cast<unsigned>(write_grad ? a.S : 1));
  if (dtype == 0)
    hipLaunchKernelGGL(ce_grad_kernel<float>, grid, dim3(kThreads), 0, s, a, write_grad);
  else
    hipLaunchKernelGGL(ce_grad_kernel<uint16_t>, grid, dim3(kThreads), 0, s, a, write_grad);
  return hipGetLastError();
}

hipError_t launch_loss_reduce_dev(const float* row_loss, int64_t n, const float* scale,
                                  float* loss, hipStream_t s) {
  hipLaunchKernelGGL(loss_reduce_dev_kernel, dim3(1), dim3(kReduceThreads), 0, s, row_loss, n,
                     scale, loss);
  return hipGetLastError();
}

}  // namespace fljsd
