// bf16 transpose: dst[c][r] = src[r][c]. The weight-gradient product
// grad_W = dZ^T X_s (Liger-Kernel PR #1429, Summary) reads both operands with
// the reduction index (the chunk's rows) fastest once dZ and X_s are
// transposed, so it runs on the matrix-core path whose operands are copied
// straight from global memory into LDS. The copy is HBM-bound: one read and
// one write of each element.
//
// A 256-thread workgroup moves a 64 x 64 tile through LDS. Global reads and
// writes are 16-byte vectors, eight threads per 128-byte row segment. The LDS
// tile keeps 16-byte chunks XOR-swizzled by row / 8 so that both the row-wise
// writes and the column-wise reads are free of bank conflicts.
#include "kernels.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fljsd {
namespace {

constexpr int kT = 64;      // tile edge
constexpr int kThreads = 256;

__device__ inline int tswz(int row, int chunk) { return chunk ^ ((row >> 3) & 7); }

__global__ __launch_bounds__(kThreads) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                                  int64_t rows, int64_t cols,
                                                                  int64_t ld_src,
                                                                  uint16_t* __restrict__ dst,
                                                                  int64_t ld_dst, bool vec_src,
                                                                  bool vec_dst, int64_t tiles_c) {
  __shared__ uint4 tile[kT][kT / 8];
  const int tid = threadIdx.x;
  const int64_t r0 = (blockIdx.x / tiles_c) * kT;
  const int64_t c0 = (blockIdx.x % tiles_c) * kT;

  // Load: thread -> (row, 16-byte chunk); two passes of 32 rows.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = tid / 8 + 32 * h;
    const int chunk = tid % 8;
    const int64_t r = r0 + row;
    const int64_t c = c0 + chunk * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < rows) {
      const uint16_t* p = src + r * ld_src + c;
      if (vec_src && c + 8 <= cols) {
        v = *reinterpret_cast<const uint4*>(p);
      } else {
        uint16_t e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = c + k < cols ? p[k] : uint16_t(0);
        v = make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                       e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
      }
    }
    tile[row][tswz(row, chunk)] = v;
  }
  __syncthreads();

  // Store: thread -> (source column, eight consecutive source rows); a wave
  // writes 8 destination rows of 128 contiguous bytes. Two passes of 32 columns.
  const uint16_t* t16 = reinterpret_cast<const uint16_t*>(&tile[0][0]);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col = tid / 8 + 32 * h;
    const int j = tid % 8;
    const int64_t c = c0 + col;
    if (c >= cols) continue;
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * j + i;
      e[i] = t16[row * kT + tswz(row, col >> 3) * 8 + (col & 7)];
    }
    const int64_t r = r0 + 8 * j;
    uint16_t* q = dst + c * ld_dst + r;
    if (vec_dst && r + 8 <= rows) {
      *reinterpret_cast<uint4*>(q) =
          make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                     e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (r + i < rows) q[i] = e[i];
    }
  }
}

}  // namespace

hipError_t launch_transpose_bf16(const void* src, int64_t rows, int64_t cols, int64_t ld_src,
                                 void* dst, int64_t ld_dst, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t tiles_r = (rows + kT - 1) / kT;
  const int64_t tiles_c = (cols + kT - 1) / kT;
  const bool vec_src = (ld_src % 8) == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  const bool vec_dst = (ld_dst % 8) == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(static_cast<unsigned>(tiles_r * tiles_c)),
                     dim3(kThreads), 0, s, static_cast<const uint16_t*>(src), rows, cols, ld_src,
                     static_cast<uint16_t*>(dst), ld_dst, vec_src, vec_dst, tiles_c);
  return hipGetLastError();
}

}  // namespace fljsd
