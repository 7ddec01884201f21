// bf16 GEMMs on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16), fp32
// accumulation, one rounding to bf16 at the end (Liger-Kernel PR #1352,
// Details: the GEMM keeps the input dtype; PR #1429, Summary: the product and
// beta*C are added in fp32 and rounded once).
//
// One kernel template serves the pass's three products:
//   logits       Z[C,V]    = X[C,H] W[V,H]^T     A and B K-contiguous
//   grad_input   gX[C,H]   = dZ[C,V] W[V,H]      A K-contiguous, B N-contiguous
//   grad_weight  gW[V,H] (+)= dZ[C,V]^T X[C,H]   A M-contiguous, B N-contiguous
// LDS always holds both operands K-contiguous ([row][k], 64 k per row, 16-byte
// chunks XOR-swizzled), so the matrix-core loop is shared. A K-contiguous
// operand is copied 16 bytes at a time; an M/N-contiguous one is read as
// 8 (m) x 4 (k) blocks of four 16-byte row segments and transposed in
// registers into 8-byte LDS writes.
//
// Pipeline: two LDS stages; the next K-tile's global loads are issued before
// the current tile's MFMAs and written to the other stage after them, with one
// barrier per K-tile.
#include "kernels.h"
#include "plan.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fljsd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BK = kGemmBK;       // K per LDS stage
constexpr int CPR = BK / 8;       // 16-byte chunks per LDS row

// Physical chunk of logical chunk c in LDS row r. Rows r..r+7 (an MFMA
// fragment read) and rows 8j+i for consecutive j (a transposed write) each
// land on 8 distinct chunks.
__device__ inline int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

__device__ inline uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline uint4 load_partial_row(const uint16_t* p, int n) {
  // n in [0, 8): elements past n read as zero.
  uint16_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = i < n ? p[i] : uint16_t(0);
  return make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                    e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool A_K, bool B_K, int EPI>
struct GemmKernel {
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int TM = WM / 32;
  static constexpr int TN = WN / 32;
  // 32-element load units per thread per operand and K-tile.
  static constexpr int UA = BM * BK / (NT * 32);
  static constexpr int UB = BN * BK / (NT * 32);
  static_assert(UA >= 1 && UA * NT * 32 == BM * BK, "A tile must split evenly");
  static_assert(UB >= 1 && UB * NT * 32 == BN * BK, "B tile must split evenly");
  static_assert(TM >= 1 && TN >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile");
  static constexpr int LDS_STAGE = (BM + BN) * CPR;   // uint4 per stage

  // Global -> registers for one operand tile of R rows (M or N side).
  template <int R, int U, bool KCONTIG>
  static __device__ inline void load_tile(const uint16_t* __restrict__ p, int64_t ld,
                                          int64_t row0, int64_t dim, int64_t k0, int64_t kend,
                                          uint4* reg) {
    const int tid = threadIdx.x;
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < 4 * U; ++i) {
        const int cid = tid + i * NT;
        const int r = cid / CPR;
        const int ch = cid % CPR;
        const int64_t row = row0 + r;
        const int64_t k = k0 + ch * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < dim && k < kend) {
          const uint16_t* src = p + row * ld + k;
          if (k + 8 <= kend)
            v = *reinterpret_cast<const uint4*>(src);
          else
            v = load_partial_row(src, static_cast<int>(kend - k));
        }
        reg[i] = v;
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int uid = tid + u * NT;
        const int mb = uid % (R / 8);
        const int kq = uid / (R / 8);
        const int64_t mn = row0 + mb * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t k = k0 + kq * 4 + q;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (k < kend && mn < dim) {
            const uint16_t* src = p + k * ld + mn;
            if (mn + 8 <= dim)
              v = *reinterpret_cast<const uint4*>(src);
            else
              v = load_partial_row(src, static_cast<int>(dim - mn));
          }
          reg[u * 4 + q] = v;
        }
      }
    }
  }

  // Registers -> LDS stage (rows [0, R) of the operand region at `base`).
  template <int R, int U, bool KCONTIG>
  static __device__ inline void store_tile(uint4* lds, int base_row, const uint4* reg) {
    const int tid = threadIdx.x;
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < 4 * U; ++i) {
        const int cid = tid + i * NT;
        const int r = cid / CPR;
        const int ch = cid % CPR;
        lds[(base_row + r) * CPR + swz(r, ch)] = reg[i];
      }
    } else {
      uint2* lds2 = reinterpret_cast<uint2*>(lds);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int uid = tid + u * NT;
        const int mb = uid % (R / 8);
        const int kq = uid / (R / 8);
        const uint4 v0 = reg[u * 4 + 0], v1 = reg[u * 4 + 1];
        const uint4 v2 = reg[u * 4 + 2], v3 = reg[u * 4 + 3];
        const uint32_t a0[4] = {v0.x, v0.y, v0.z, v0.w};
        const uint32_t a1[4] = {v1.x, v1.y, v1.z, v1.w};
        const uint32_t a2[4] = {v2.x, v2.y, v2.z, v2.w};
        const uint32_t a3[4] = {v3.x, v3.y, v3.z, v3.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int d = i >> 1;
          uint2 w;
          if ((i & 1) == 0) {
            w.x = (a0[d] & 0xffffu) | (a1[d] << 16);
            w.y = (a2[d] & 0xffffu) | (a3[d] << 16);
          } else {
            w.x = (a0[d] >> 16) | (a1[d] & 0xffff0000u);
            w.y = (a2[d] >> 16) | (a3[d] & 0xffff0000u);
          }
          const int r = mb * 8 + i;
          lds2[((base_row + r) * CPR + swz(r, kq >> 1)) * 2 + (kq & 1)] = w;
        }
      }
    }
  }

  static __device__ void run(const GemmArgs& g, int tiles_m) {
    __shared__ uint4 lds[2][LDS_STAGE];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_m = wave % WAVES_M;
    const int wave_n = wave / WAVES_M;

    const int64_t bid = blockIdx.x;
    const int64_t tm = bid % tiles_m;
    const int64_t tn = bid / tiles_m;
    const int64_t m0 = tm * BM;
    const int64_t n0 = tn * BN;
    const int split = blockIdx.y;
    const int64_t kb = static_cast<int64_t>(split) * g.k_per_split;
    const int64_t ke = min(g.K, kb + g.k_per_split);
    const int nk = static_cast<int>((ke - kb + BK - 1) / BK);

    const uint16_t* A = static_cast<const uint16_t*>(g.A);
    const uint16_t* B = static_cast<const uint16_t*>(g.B);

    floatx16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    uint4 ra[4 * UA], rb[4 * UB];
    load_tile<BM, UA, A_K>(A, g.lda, m0, g.M, kb, ke, ra);
    load_tile<BN, UB, B_K>(B, g.ldb, n0, g.N, kb, ke, rb);
    store_tile<BM, UA, A_K>(lds[0], 0, ra);
    store_tile<BN, UB, B_K>(lds[0], BM, rb);
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
      const bool more = t + 1 < nk;
      if (more) {
        const int64_t k0 = kb + static_cast<int64_t>(t + 1) * BK;
        load_tile<BM, UA, A_K>(A, g.lda, m0, g.M, k0, ke, ra);
        load_tile<BN, UB, B_K>(B, g.ldb, n0, g.N, k0, ke, rb);
      }
      const uint4* cur = lds[t & 1];
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int ch = ks * 2 + (lane >> 5);
        bf16x8 fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int r = wave_m * WM + i * 32 + (lane & 31);
          fa[i] = __builtin_bit_cast(bf16x8, cur[r * CPR + swz(r, ch)]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int r = wave_n * WN + j * 32 + (lane & 31);
          fb[j] = __builtin_bit_cast(bf16x8, cur[(BM + r) * CPR + swz(r, ch)]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      if (more) {
        store_tile<BM, UA, A_K>(lds[(t + 1) & 1], 0, ra);
        store_tile<BN, UB, B_K>(lds[(t + 1) & 1], BM, rb);
      }
      __syncthreads();
    }

    // Epilogue. Accumulator register r of lane l in a 32x32 tile holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wave_n * WN + j * 32 + (lane & 31);
        if (n >= g.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wave_m * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (m >= g.M) continue;
          const float v = acc[i][j][r];
          if constexpr (EPI == kEpiPartialF32) {
            float* C = static_cast<float*>(g.C) + static_cast<int64_t>(split) * g.M * g.ldc;
            C[m * g.ldc + n] = v;
          } else {
            uint16_t* C = static_cast<uint16_t*>(g.C);
            float out = v;
            if constexpr (EPI == kEpiAccumulate)
              out += __uint_as_float(static_cast<uint32_t>(C[m * g.ldc + n]) << 16);
            C[m * g.ldc + n] = static_cast<uint16_t>(f32_to_bf16_bits(out));
          }
        }
      }
    }
  }
};

template <int BM, int BN, int WAVES_M, int WAVES_N, bool A_K, bool B_K, int EPI>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void gemm_bf16_kernel(GemmArgs g,
                                                                           int tiles_m) {
  GemmKernel<BM, BN, WAVES_M, WAVES_N, A_K, B_K, EPI>::run(g, tiles_m);
}

constexpr int kWavesM = 2;
constexpr int kWavesN = 4;

template <bool A_K, bool B_K, int EPI>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  const int64_t tiles_m = (g.M + kGemmBM - 1) / kGemmBM;
  const int64_t tiles_n = (g.N + kGemmBN - 1) / kGemmBN;
  const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n), static_cast<unsigned>(g.splitk));
  const dim3 block(kWavesM * kWavesN * 64);
  hipLaunchKernelGGL((gemm_bf16_kernel<kGemmBM, kGemmBN, kWavesM, kWavesN, A_K, B_K, EPI>),
                     grid, block, 0, s, g, static_cast<int>(tiles_m));
  return hipGetLastError();
}

template <bool A_K, bool B_K>
hipError_t launch_layout(const GemmArgs& g, hipStream_t s) {
  switch (g.epilogue) {
    case kEpiStore: return launch_cfg<A_K, B_K, kEpiStore>(g, s);
    case kEpiAccumulate: return launch_cfg<A_K, B_K, kEpiAccumulate>(g, s);
    default: return launch_cfg<A_K, B_K, kEpiPartialF32>(g, s);
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  // The three layouts the pass uses.
  if (g.a_kcontig && g.b_kcontig) return launch_layout<true, true>(g, s);
  if (g.a_kcontig && !g.b_kcontig) return launch_layout<true, false>(g, s);
  if (!g.a_kcontig && !g.b_kcontig) return launch_layout<false, false>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace fljsd
