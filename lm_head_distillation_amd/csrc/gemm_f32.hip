// fp32 GEMMs for fp32 inputs: true fp32 products and sums (no reduced-precision
// matrix-core path), so the fp32 pass keeps fp32 accuracy end to end. Same
// three operand layouts and epilogues as the bf16 kernels. A 64x64 output tile
// per 256-thread workgroup, 4x4 outputs per thread, operands staged through LDS.
#include "kernels.h"
#include "plan.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fljsd {
namespace {

constexpr int BM = kGemmF32BM;
constexpr int BN = kGemmF32BN;
constexpr int BKF = 16;
constexpr int NT = 256;

template <int EPI>
__global__ __launch_bounds__(NT) void gemm_f32_kernel(GemmArgs g, int tiles_m) {
  __shared__ float As[BKF][BM + 4];
  __shared__ float Bs[BKF][BN + 4];
  const float* A = static_cast<const float*>(g.A);
  const float* B = static_cast<const float*>(g.B);
  // Element strides: A(m,k) = A[m*sam + k*sak], B(n,k) = B[n*sbn + k*sbk].
  const int64_t sam = g.a_kcontig ? g.lda : 1;
  const int64_t sak = g.a_kcontig ? 1 : g.lda;
  const int64_t sbn = g.b_kcontig ? g.ldb : 1;
  const int64_t sbk = g.b_kcontig ? 1 : g.ldb;

  const int tid = threadIdx.x;
  const int64_t bid = blockIdx.x;
  const int64_t m0 = (bid % tiles_m) * BM;
  const int64_t n0 = (bid / tiles_m) * BN;
  const int split = blockIdx.y;
  const int64_t kb = static_cast<int64_t>(split) * g.k_per_split;
  const int64_t ke = min(g.K, kb + g.k_per_split);
  const int tx = tid % 16;  // n direction
  const int ty = tid / 16;  // m direction

  float acc[4][4] = {};
  for (int64_t k0 = kb; k0 < ke; k0 += BKF) {
    // Each operand tile is BKF x 64 = 1024 elements: 4 per thread.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * NT;
      int kk, mm;
      if (g.a_kcontig) {
        kk = e % BKF;
        mm = e / BKF;
      } else {
        mm = e % BM;
        kk = e / BM;
      }
      const int64_t m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < g.M && k < ke) ? A[m * sam + k * sak] : 0.f;
      int kn, nn;
      if (g.b_kcontig) {
        kn = e % BKF;
        nn = e / BKF;
      } else {
        nn = e % BN;
        kn = e / BN;
      }
      const int64_t n = n0 + nn, kb2 = k0 + kn;
      Bs[kn][nn] = (n < g.N && kb2 < ke) ? B[n * sbn + kb2 * sbk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKF; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n >= g.N) continue;
      float* C = static_cast<float*>(g.C);
      if constexpr (EPI == kEpiPartialF32) {
        C[static_cast<int64_t>(split) * g.M * g.ldc + m * g.ldc + n] = acc[i][j];
      } else if constexpr (EPI == kEpiAccumulate) {
        C[m * g.ldc + n] += acc[i][j];
      } else {
        C[m * g.ldc + n] = acc[i][j];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s) {
  const int64_t tiles_m = (g.M + BM - 1) / BM;
  const int64_t tiles_n = (g.N + BN - 1) / BN;
  const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n), static_cast<unsigned>(g.splitk));
  switch (g.epilogue) {
    case kEpiStore:
      hipLaunchKernelGGL(gemm_f32_kernel<kEpiStore>, grid, dim3(NT), 0, s, g,
                         static_cast<int>(tiles_m));
      break;
    case kEpiAccumulate:
      hipLaunchKernelGGL(gemm_f32_kernel<kEpiAccumulate>, grid, dim3(NT), 0, s, g,
                         static_cast<int>(tiles_m));
      break;
    default:
      hipLaunchKernelGGL(gemm_f32_kernel<kEpiPartialF32>, grid, dim3(NT), 0, s, g,
                         static_cast<int>(tiles_m));
      break;
  }
  return hipGetLastError();
}

}  // namespace fljsd
