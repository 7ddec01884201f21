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

#include <algorithm>
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
    load8<false>(z, v, n, a.vec_ok, x);
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
    load8<false>(z, v, n, a.vec_ok, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = hw_exp2((x[i] - m) * kLog2e - l2d);
      const float dz = q - off - (v + i == y ? hit : 0.f);
      out[i] = ok ? dz * gs : 0.f;
    }
    store8<false>(gr, v, n, a.vec_ok, out);
  }
}

// Pass 2 over 64-row x 64-column tiles, bf16, for a weight-gradient product:
// dZ written in place as by ce_grad_kernel and the same tile, transposed
// through LDS (16-byte chunk c of row r at c ^ ((r / 8) % 8)), to dzt [V, ldt].
// A workgroup covers 64 rows and `span` columns; threads 0..63 first merge
// their row's statistics and write its loss.
constexpr int64_t kTileColsMax = 1024;
constexpr int64_t kGradTargetBlocks = 2048;

__global__ __launch_bounds__(kThreads) void ce_grad_t_kernel(CeArgs a, uint16_t* dzt, int64_t ldt,
                                                            int64_t span) {
  __shared__ float2 sh_ml[64];   // (m, log2 d)
  __shared__ float sh_gs[64];    // gradient scale of the row (0 when it does not count)
  __shared__ int64_t sh_y[64];
  __shared__ uint4 tile[64][8];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int64_t c_begin = static_cast<int64_t>(blockIdx.x) * span;
  const int64_t c_end = min(a.V, c_begin + span);
  const int t = threadIdx.x;
  const float Vf = static_cast<float>(a.V);
  if (t < 64) {
    const int64_t row = r0 + t;
    float2 ml = make_float2(0.f, 0.f);
    float gs = 0.f;
    int64_t y = -1;
    if (row < a.rows) {
      const float4* st = a.stats + row * a.S;
      float4 acc = st[0];
      for (int j = 1; j < a.S; ++j) {
        md_merge(acc.x, acc.y, st[j].x, st[j].y, kLog2e);
        acc.z += st[j].z;
      }
      ml = make_float2(acc.x, hw_log2(acc.y));
      y = a.labels[row];
      const bool ok = counted(y, a.V, a.ignore_index);
      gs = ok ? a.scale[0] : 0.f;
      if (blockIdx.x == 0) {
        const float lse = acc.x + ml.y * 0.693147180559945309f;
        a.row_loss[row] = ok ? lse - (1.f - a.eps) * a.zy[row] - (a.eps / Vf) * acc.z : 0.f;
      }
    }
    sh_ml[t] = ml;
    sh_gs[t] = gs;
    sh_y[t] = y;
  }
  __syncthreads();
  const uint16_t* z = static_cast<const uint16_t*>(a.z);
  uint16_t* gr = static_cast<uint16_t*>(a.grad);
  const float off = a.eps / Vf;
  const float hit = 1.f - a.eps;
  for (int64_t c0 = c_begin; c0 < c_end; c0 += 64) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rl = t / 8 + 32 * h;
      const int chunk = t % 8;
      const int64_t row = r0 + rl;
      const int64_t v = c0 + chunk * 8;
      uint4 packed = make_uint4(0, 0, 0, 0);
      if (row < a.rows && v < a.V) {
        const int n = static_cast<int>(min<int64_t>(8, a.V - v));
        const float2 ml = sh_ml[rl];
        const float gs = sh_gs[rl];
        const int64_t y = sh_y[rl];
        float x[8], out[8];
        load8<false>(z + row * a.ld, v, n, a.vec_ok, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float q = hw_exp2((x[i] - ml.x) * kLog2e - ml.y);
          out[i] = (q - off - (v + i == y ? hit : 0.f)) * gs;
        }
        packed = pack8_bf16(out, n);
        store8_packed<false>(gr + row * a.ld, v, n, a.vec_ok, packed);
      }
      tile[rl][chunk ^ ((rl >> 3) & 7)] = packed;
    }
    __syncthreads();
    const uint16_t* t16 = reinterpret_cast<const uint16_t*>(&tile[0][0]);
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
          *reinterpret_cast<uint4*>(q) =
              make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                         e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
        } else {
          for (int i = 0; i < 8; ++i)
            if (r + i < a.rows) q[i] = e[i];
        }
      }
    }
    __syncthreads();
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

hipError_t launch_ce_grad_transposed(const CeArgs& a, void* dzt, int64_t ldt, hipStream_t s) {
  const int64_t row_blocks = (a.rows + 63) / 64;
  const int64_t tiles = (a.V + 63) / 64;
  int64_t per = (tiles * row_blocks + kGradTargetBlocks - 1) / kGradTargetBlocks;
  per = std::max<int64_t>(1, std::min<int64_t>(per, kTileColsMax / 64));
  const int64_t span = per * 64;
  const dim3 grid(static_cast<unsigned>((a.V + span - 1) / span), static_cast<unsigned>(row_blocks));
  hipLaunchKernelGGL(ce_grad_t_kernel, grid, dim3(kThreads), 0, s, a, static_cast<uint16_t*>(dzt),
                     ldt, span);
  return hipGetLastError();
}

hipError_t launch_loss_reduce_dev(const float* row_loss, int64_t n, const float* scale,
                                  float* loss, hipStream_t s) {
  hipLaunchKernelGGL(loss_reduce_dev_kernel, dim3(1), dim3(kReduceThreads), 0, s, row_loss, n,
                     scale, loss);
  return hipGetLastError();
}

}  // namespace fljsd
