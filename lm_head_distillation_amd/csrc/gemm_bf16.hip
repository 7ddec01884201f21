// bf16 GEMMs on CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16 on 256-row
// tiles, v_mfma_f32_32x32x16_bf16 on the skinny ones), fp32
// accumulation, one rounding to bf16 at the end (Liger-Kernel PR #1352,
// Details: the GEMM keeps the input dtype; PR #1429, Summary: the product and
// beta*C are added in fp32 and rounded once).
//
// One kernel template serves the pass's three products:
//   logits       Z[C,V]    = X[C,H] W[V,H]^T       A and B K-contiguous
//   grad_input   gX[C,H]   = dZ[C,V] W[V,H]        A K-contiguous, B N-contiguous
//                (or B = W^T, K-contiguous, when the logits product wrote it)
//   grad_weight  gW[V,H] (+)= dZ^T[V,C] X^T[H,C]^T  A and B K-contiguous (the
//                pass transposes dZ and X first; its own kernel symbol)
// LDS always holds both operands K-contiguous ([row][k], 16-byte chunks
// XOR-swizzled so fragment reads are bank-conflict free), so the matrix-core
// loop is shared. A K-contiguous operand of a block inside the operands is
// copied straight from global memory into LDS (gfx950 global_load_lds_dwordx4,
// no registers); an N-contiguous one is read as 8 (n) x 4 (k) blocks of four
// 16-byte row segments and transposed in registers into 8-byte LDS writes.
//
// Pipeline: K-tiles of 64 (128-byte rows, whole cache lines) through two LDS
// stages. The two waves
// sharing a SIMD issue the next tile's loads at different K steps, so one
// keeps the matrix core busy while the other waits for its loads to be
// accepted; on 256 x 256 tiles the later of the two issues fewer of them.
// Edge blocks and a partial last K-tile take a bounds-checked
// register path. Within a stage the source reads each K step's fragments
// ahead of the previous step's MFMAs (16 x 16 tiles: the next step's B
// fragments ahead, each A fragment again once its row of products has
// issued); the compiler moves the reads next to their MFMAs, and the SIMD's
// other wave covers the LDS latency.
// Workgroups are renumbered so the tiles
// one XCD runs together share operand panels in that XCD's L2. Epilogues:
// store (bf16), fp32 store (split-K partials, fp32 weight gradient), and
// read-add-write in bf16 or fp32 for the weight gradient of later chunks.
#include "elem_math.h"
#include "kernels.h"
#include "plan.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <cstdint>

namespace fljsd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Matrix-core instruction: v_mfma_f32_16x16x32_bf16 (16 x 16 outputs, 32-deep
// products) or v_mfma_f32_32x32x16_bf16. Both have the same nominal rate, but
// in a register-only loop with random operands on every CU the 16 x 16 form
// sustains 91% of it against 80% for the 32 x 32 form. The 256-row tiles use
// the 16 x 16 form (the pass at 8192 x 4096 x 128256: 31.8 -> 30.2 ms); the
// skinny tiles of small chunks, which stream the weights, keep 32 x 32 (16 x
// 16 made them 10-15% slower).
template <int MS> struct Mfma;
template <> struct Mfma<32> {
  using Acc = floatx16;
  static constexpr int K = 16;
  static __device__ inline Acc run(bf16x8 a, bf16x8 b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<16> {
  using Acc = floatx4;
  static constexpr int K = 32;
  static __device__ inline Acc run(bf16x8 a, bf16x8 b, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;  // MI355X: workgroups go round-robin to 8 XCDs, each with its own L2

// Output tile of workgroup `bid`. Workgroup ids are first renumbered so each
// XCD receives one contiguous range of logical ids (the hardware deals ids
// out round-robin across XCDs), then logical ids walk the tiles in groups of
// `group_m` M-tiles: M fastest within a group, then N, then the next group.
// Tiles that run together on one XCD therefore share operand panels in its L2.
__device__ inline void tile_of(int bid, int nblk, int tiles_m, int tiles_n, int group_m, int& tm,
                               int& tn) {
  const int xcd = bid % kXcds;
  const int per = nblk / kXcds;
  const int rem = nblk % kXcds;
  const int logical = xcd * per + min(xcd, rem) + bid / kXcds;
  const int in_group = group_m * tiles_n;
  const int first_m = (logical / in_group) * group_m;
  const int gm = min(group_m, tiles_m - first_m);
  const int r = logical % in_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

// The M-tile whose workgroup writes B^T for N-tile tn (GemmArgs::bt): one of
// the whole M-tiles, rotating with tn. Each XCD runs one range of M-tile
// groups (tile_of), so a fixed M-tile would put every writer, and all of the
// B^T stores, on one XCD.
__device__ inline int side_tile_m(const GemmArgs& g, int tn) {
  return tn % static_cast<int>(g.M / kGemmBM);
}

// Physical 16-byte chunk of logical chunk c in LDS row r (eight chunks, 128
// bytes, per row). Eight rows' chunk c (one fragment read of eight lanes)
// land in eight distinct bank groups, and so do the transposed writes of rows
// 8j + i for consecutive j.
template <int CPR>
__device__ inline int swz(int r, int c) {
  static_assert(CPR == 8, "64-wide K-tiles");
  return c ^ ((r ^ (r >> 3)) & 7);
}

// A lane's value after a DPP move within its 16-lane row (gfx9 encodings):
// quad_perm [1,0,3,2] and [2,3,0,1] exchange with lane ^ 1 and lane ^ 2,
// row_half_mirror pairs lane i with 7 - i in each group of eight, row_mirror
// i with 15 - i in the row. Each reads a lane of the same row, so no lane is
// out of range and bound_ctrl changes nothing; with it the move needs no old
// value (no zeroed register before each move, and adds fuse into
// v_add_f32_dpp).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Max and sum over a 32-lane half-wave, as butterflies: after each step both
// partners hold the same value (max and two-term sums are commutative), so
// mirror partners serve as well as xor partners. Every lane ends with the
// result.
__device__ inline float half_wave_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  x = fmaxf(x, dpp<kDppMirror>(x));
  return fmaxf(x, __shfl_xor(x, 16, 64));
}
__device__ inline float half_wave_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return x + __shfl_xor(x, 16, 64);
}

__device__ inline uint4 load_partial_row(const uint16_t* p, int n) {
  // n in [0, 8): elements past n read as zero.
  uint16_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = i < n ? p[i] : uint16_t(0);
  return make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                    e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
}

// Wait for all of this wave's outstanding vector-memory loads (a direct
// copy counts until its data is in LDS).
__device__ inline void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int BM, int BN, int BK, int STAGES, int WAVES_M, int WAVES_N, bool A_K, bool B_K,
          int EPI, bool PRE_OLD = false, int EARLY_B = -1, bool SIDE = false>
struct GemmKernel {
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int NW = NT / 64;
  static constexpr int CPR = BK / 8;               // 16-byte chunks per LDS row
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  // Matrix-core tiles of MS x MS outputs; a lane holds NACC accumulators of
  // each, in groups of four consecutive rows (or, transposed, columns).
  static constexpr int MS = BM >= 256 ? 16 : 32;
  using Acc = typename Mfma<MS>::Acc;
  static constexpr int NACC = MS * MS / 64;
  static constexpr int KSTEP = Mfma<MS>::K;
  static constexpr int TM = WM / MS;
  static constexpr int TN = WN / MS;
  static constexpr int LDS_STAGE = (BM + BN) * CPR;   // uint4 per stage
  static_assert(CPR == 8, "K-tile of 64");
  static_assert(TM >= 1 && TN >= 1 && WM % MS == 0 && WN % MS == 0, "wave tile");
  static_assert(STAGES == 2, "two LDS stages of 64-wide K-tiles");
  // The staged epilogues compute the transposed products (B's fragment
  // first), which leaves four consecutive output columns of one row in each
  // group of four accumulator registers: a lane's four columns go to LDS as
  // one 8-byte (bf16) or 16-byte (fp32) write.
  static constexpr bool SWAP_D = EPI == kEpiAccumulate || EPI == kEpiAccumulateF32 ||
                                 EPI == kEpiStore || EPI == kEpiStoreStats;
  static_assert(!SWAP_D || STAGES * LDS_STAGE * 16 >= BM * BN * 2,
                "the staged epilogue holds the whole bf16 tile in LDS");

  // Register path: a K-contiguous tile of R rows moves in 16-byte chunks,
  // chunks(R) per thread; an M/N-contiguous one in 8 x 4 blocks, units(R) per
  // thread (each four 16-byte loads).
  static constexpr int chunks(int R) { return R * CPR / NT; }
  static constexpr int units(int R) { return R * BK / (NT * 32); }
  static constexpr int regs(int R, bool kcontig) { return kcontig ? chunks(R) : 4 * units(R); }
  // Direct copies: one wave instruction fills 64 / CPR rows (1 KB).
  static constexpr int dma_insts(int R) { return R / (64 / CPR) / NW; }

  template <int R, bool KCONTIG>
  static __device__ inline void check_split() {
    if constexpr (KCONTIG)
      static_assert(chunks(R) >= 1 && chunks(R) * NT == R * CPR, "tile must split evenly");
    else
      static_assert(units(R) >= 1 && units(R) * NT * 32 == R * BK, "tile must split evenly");
  }

  // Global -> registers, bounds-checked (rows past `dim`, K past `kend` read 0).
  template <int R, bool KCONTIG>
  static __device__ inline void load_tile(const uint16_t* __restrict__ p, int64_t ld,
                                          int64_t row0, int64_t dim, int64_t k0, int64_t kend,
                                          uint4* reg) {
    check_split<R, KCONTIG>();
    const int tid = threadIdx.x;
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < chunks(R); ++i) {
        const int cid = tid + i * NT;
        const int64_t row = row0 + cid / CPR;
        const int64_t k = k0 + (cid % CPR) * 8;
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
      for (int u = 0; u < units(R); ++u) {
        const int uid = tid + u * NT;
        const int64_t mn = row0 + (uid % (R / 8)) * 8;
        const int64_t kk = k0 + (uid / (R / 8)) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t k = kk + q;
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

  // Global -> registers for a tile that lies wholly inside the operand.
  template <int R, bool KCONTIG>
  static __device__ inline void load_tile_fast(const uint16_t* __restrict__ p, int64_t ld,
                                               int64_t row0, int64_t k0, uint4* reg) {
    check_split<R, KCONTIG>();
    const int tid = threadIdx.x;
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < chunks(R); ++i) {
        const int cid = tid + i * NT;
        reg[i] = *reinterpret_cast<const uint4*>(p + (row0 + cid / CPR) * ld + k0 + (cid % CPR) * 8);
      }
    } else {
#pragma unroll
      for (int u = 0; u < units(R); ++u) {
        const int uid = tid + u * NT;
        const int64_t mn = row0 + (uid % (R / 8)) * 8;
        const int64_t kk = k0 + (uid / (R / 8)) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          reg[u * 4 + q] = *reinterpret_cast<const uint4*>(p + (kk + q) * ld + mn);
      }
    }
  }

  // Registers -> LDS rows [base_row, base_row + R) of `stage`.
  template <int R, bool KCONTIG>
  static __device__ inline void store_tile(uint4* stage, int base_row, const uint4* reg) {
    const int tid = threadIdx.x;
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < chunks(R); ++i) {
        const int cid = tid + i * NT;
        const int r = cid / CPR;
        stage[(base_row + r) * CPR + swz<CPR>(r, cid % CPR)] = reg[i];
      }
    } else {
      uint2* lds2 = reinterpret_cast<uint2*>(stage);
#pragma unroll
      for (int u = 0; u < units(R); ++u) {
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
          lds2[((base_row + r) * CPR + swz<CPR>(r, kq >> 1)) * 2 + (kq & 1)] = w;
        }
      }
    }
  }

  // Direct global -> LDS copy of a K-contiguous tile of R rows (interior,
  // whole K-tile). Lane l of an instruction lands in LDS slot l, i.e. row
  // l / CPR at physical chunk l % CPR, so it loads the logical chunk the
  // swizzle maps there (the swizzle is an XOR, its own inverse).
  template <int R>
  static __device__ inline void dma_tile(const uint16_t* __restrict__ p, int64_t ld,
                                         int64_t row0, int64_t k0, uint4* region) {
    constexpr int ROWS = 64 / CPR;
    static_assert(dma_insts(R) * NW * ROWS == R, "rows must split evenly over the waves");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < dma_insts(R); ++i) {
      const int rb = (wave + i * NW) * ROWS;   // first row this instruction fills
      const int r = rb + lane / CPR;
      const int c = swz<CPR>(r, lane % CPR);
      const uint16_t* src = p + (row0 + r) * ld + k0 + c * 8;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(region + rb * CPR), 16, 0, 0);
    }
  }

  // Rows [r_begin, r_begin + 32 * NINST) of a K-contiguous tile, copied by the
  // four waves of one half of the workgroup (wg = this wave's index in it).
  template <int NINST>
  static __device__ inline void dma_rows(const uint16_t* __restrict__ p, int64_t ld, int64_t row0,
                                         int64_t k0, uint4* region, int r_begin, int wg) {
    constexpr int ROWS = 64 / CPR;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NINST; ++i) {
      const int rb = r_begin + (wg + i * 4) * ROWS;   // first row this instruction fills
      const int r = rb + lane / CPR;
      const int c = swz<CPR>(r, lane % CPR);
      const uint16_t* src = p + (row0 + r) * ld + k0 + c * 8;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(region + rb * CPR), 16, 0, 0);
    }
  }

  // Fragments of one K step (KSTEP deep) for this wave: lane l reads row
  // l % MS of each tile, 16 bytes at K offset 8 (l / MS).
  static __device__ inline bf16x8 frag_a(const uint4* cur, int ks, int lane, int wave_m, int i) {
    const int ch = ks * (KSTEP / 8) + lane / MS;
    const int r = wave_m * WM + i * MS + lane % MS;
    return __builtin_bit_cast(bf16x8, cur[r * CPR + swz<CPR>(r, ch)]);
  }
  static __device__ inline bf16x8 frag_b(const uint4* cur, int ks, int lane, int wave_n, int j) {
    const int ch = ks * (KSTEP / 8) + lane / MS;
    const int r = wave_n * WN + j * MS + lane % MS;
    return __builtin_bit_cast(bf16x8, cur[(BM + r) * CPR + swz<CPR>(r, ch)]);
  }
  static __device__ inline void read_frags(const uint4* cur, int ks, int lane, int wave_m,
                                           int wave_n, bf16x8* fa, bf16x8* fb) {
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = frag_a(cur, ks, lane, wave_m, i);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = frag_b(cur, ks, lane, wave_n, j);
  }
  // Accumulator group q (four registers) of lane l covers four consecutive
  // rows (columns, transposed) of its tile starting at quad_col(l, q).
  static __device__ inline int quad_col(int lane, int q) { return 4 * (lane / MS) + (256 / MS) * q; }
  static __device__ inline Acc mma(bf16x8 a, bf16x8 b, Acc c) {
    // SWAP_D: the transposed product (B's fragment first).
    return SWAP_D ? Mfma<MS>::run(b, a, c) : Mfma<MS>::run(a, b, c);
  }

  // MFMAs over one LDS stage, the next K step's fragments requested before
  // the current step's products (the compiler may still schedule each read
  // next to its MFMAs). hook(ks) runs before step ks's MFMAs (the main loops
  // issue the next tile's global loads from it).
  template <class Hook>
  static __device__ inline void compute_stage(const uint4* cur, Acc (&acc)[TM][TN],
                                              Hook&& hook) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wave_m = wave % WAVES_M;
    const int wave_n = wave / WAVES_M;
    constexpr int KS = BK / KSTEP;
    if constexpr (MS == 32) {
      bf16x8 fa[2][TM], fb[2][TN];
      read_frags(cur, 0, lane, wave_m, wave_n, fa[0], fb[0]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) read_frags(cur, ks + 1, lane, wave_m, wave_n, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
        hook(ks);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mma(fa[ks & 1][i], fb[ks & 1][j], acc[i][j]);
      }
    } else {
      // Twice the fragments per K step: the next step's B fragments are read
      // ahead into their own registers, each A fragment is re-read as soon as
      // its row of products has issued.
      bf16x8 fa[TM], fb[TN];
      read_frags(cur, 0, lane, wave_m, wave_n, fa, fb);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bool more = ks + 1 < KS;
        bf16x8 nb[TN];
        if (more) {
#pragma unroll
          for (int j = 0; j < TN; ++j) nb[j] = frag_b(cur, ks + 1, lane, wave_n, j);
        }
        hook(ks);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mma(fa[i], fb[j], acc[i][j]);
          if (more) fa[i] = frag_a(cur, ks + 1, lane, wave_m, i);
        }
        if (more) {
#pragma unroll
          for (int j = 0; j < TN; ++j) fb[j] = nb[j];
        }
      }
    }
  }
  static __device__ inline void compute_stage(const uint4* cur, Acc (&acc)[TM][TN]) {
    compute_stage(cur, acc, [](int) {});
  }

  // Two-stage schedules stagger the next tile's loads between the two waves
  // that share a SIMD (waves w and w + NW/2): the first half issues them
  // before K step 0, the second half before step kLateStep. While one wave
  // waits for its loads to be accepted by the memory pipeline, the other
  // keeps the SIMD's matrix core busy. Measured on the 8192 x 128256 x 4096
  // logits product: 9% faster than every wave issuing at step 0.
  static constexpr int kLateStep = BK / KSTEP / 2;
  static __device__ inline bool late_wave() { return (threadIdx.x >> 6) >= NW / 2; }

  // EARLY_B >= 0 (256 x 256 tiles, 8 waves): the early waves copy all of A
  // and the first 32 * EARLY_B rows of B, the late waves the rest of B, so
  // the late waves (whose copies are issued half a K-tile later and bound the
  // hand-off) have 8 - EARLY_B copies each instead of 8 (the loop with an
  // N-contiguous B moves only A this way). EARLY_B < 0: every wave copies
  // 1/8 of each operand.
  static constexpr bool kSplitCopies =
      EARLY_B >= 0 && EARLY_B <= 8 && BM == 256 && BN == 256 && NW == 8;

  // B^T side output (GemmArgs::bt, SIDE): the B tile of `stage` (rows n0 ..
  // n0 + BN - 1 of B, the K-tile at k0) written transposed, bt[k][n] = B(n, k).
  // gfx950's transposing LDS read (ds_read_b64_tr_b16) hands each lane four
  // consecutive rows n of one column k: in each 16-lane group, lane 4j + q
  // names row nb + 4q + j at column kb (8 bytes), and lane i receives rows
  // nb + 4(i / 4) .. + 3 of column kb + i % 4. One wave instruction covers
  // 64 rows x 4 columns, so each column's 64 rows leave as one 128-byte run.
  static constexpr bool kSideOut = SIDE;
  static_assert(!SIDE || (A_K && B_K && NW == 8 && BM == 256 && BN == 256 &&
                          (EPI == kEpiStore || EPI == kEpiStoreStats)),
                "B^T is written by the 256 x 256 tiles' direct-copy loop");
  template <int SW = NW>
  static __device__ inline void side_out(const uint4* stage, const GemmArgs& g, int64_t n0,
                                         int64_t k0) {
    const int lane = threadIdx.x & 63;
    const int wave = (threadIdx.x >> 6) % SW;
    const int grp = lane >> 4;
    const int li = lane & 15;
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const __attribute__((address_space(3))) char* base =
        (const __attribute__((address_space(3))) char*)(stage);
    uint16_t* bt = static_cast<uint16_t*>(g.bt);
    constexpr int kInst = BN * BK / (64 * 4) / SW;
#pragma unroll
    for (int u = 0; u < kInst; ++u) {
      const int idx = wave * kInst + u;
      const int nb = 64 * (idx % (BN / 64)) + 16 * grp;
      const int kb = 4 * (idx / (BN / 64));
      const int n = nb + 4 * (li & 3) + (li >> 2);
      const int off = ((BM + n) * CPR + swz<CPR>(n, kb >> 3)) * 16 + (kb & 7) * 2;
      const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + off));
      uint16_t* dst = bt + (k0 + kb + (li & 3)) * g.ldbt + n0 + nb + 4 * (li >> 2);
      *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, v);
    }
  }

  template <int STEP>
  static __device__ inline void loop_dma2(const GemmArgs& g, uint4 (*lds)[LDS_STAGE], int64_t m0,
                                          int64_t n0, int64_t kb, int nkf,
                                          Acc (&acc)[TM][TN]) {
    const uint16_t* A = static_cast<const uint16_t*>(g.A);
    const uint16_t* B = static_cast<const uint16_t*>(g.B);
    for (int t = 0; t < nkf; ++t) {
      wait_vmem_all();
      __syncthreads();
      const bool more = t + 1 < nkf;
      uint4* st = lds[(t + 1) & 1];
      const int64_t k0 = kb + static_cast<int64_t>(t + 1) * BK;
      auto issue = [&] {
        if constexpr (kSplitCopies) {
          constexpr int kEarlyB = kSplitCopies ? EARLY_B : 0;
          const int wg = (threadIdx.x >> 6) % (NW / 2);
          if constexpr (STEP == 0) {
            dma_rows<BM / 32>(A, g.lda, m0, k0, st, 0, wg);
            dma_rows<kEarlyB>(B, g.ldb, n0, k0, st + BM * CPR, 0, wg);
          } else {
            dma_rows<BN / 32 - kEarlyB>(B, g.ldb, n0, k0, st + BM * CPR, 32 * kEarlyB, wg);
          }
        } else {
          dma_tile<BM>(A, g.lda, m0, k0, st);
          dma_tile<BN>(B, g.ldb, n0, k0, st + BM * CPR);
        }
      };
      if (STEP == 0 && more) issue();
      compute_stage(lds[t & 1], acc, [&](int ks) {
        if (STEP > 0 && more && ks == STEP) issue();
      });
    }
  }

  // The workgroup that writes B^T: the early waves copy both operands, the
  // late waves write each stage's B tile transposed. Only the copying waves
  // wait for their own vector-memory operations before the hand-off barrier
  // (the writers have no copies in flight after the first tile), so the
  // writers' stores stay in flight across K-tiles.
  template <bool WRITER>
  static __device__ inline void loop_side(const GemmArgs& g, uint4 (*lds)[LDS_STAGE], int64_t m0,
                                          int64_t n0, int64_t kb, int nkf,
                                          Acc (&acc)[TM][TN]) {
    const uint16_t* A = static_cast<const uint16_t*>(g.A);
    const uint16_t* B = static_cast<const uint16_t*>(g.B);
    const int wg = (threadIdx.x >> 6) % (NW / 2);
    for (int t = 0; t < nkf; ++t) {
      if (!WRITER || t == 0) wait_vmem_all();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const bool more = t + 1 < nkf;
      if constexpr (WRITER) {
        side_out<NW / 2>(lds[t & 1], g, n0, kb + static_cast<int64_t>(t) * BK);
      } else if (more) {
        uint4* st = lds[(t + 1) & 1];
        const int64_t k0 = kb + static_cast<int64_t>(t + 1) * BK;
        dma_rows<BM / 32>(A, g.lda, m0, k0, st, 0, wg);
        dma_rows<BN / 32>(B, g.ldb, n0, k0, st + BM * CPR, 0, wg);
      }
      compute_stage(lds[t & 1], acc);
    }
  }

  // Both operands K-contiguous, interior block, whole K-tiles: every tile is
  // copied straight into LDS one tile ahead of the one multiplied. At the top
  // of iteration t, tile t's copies must have landed (each wave waits for its
  // own, the barrier for everyone's) and the other stage is free again.
  static __device__ inline void mainloop_dma(const GemmArgs& g, uint4 (*lds)[LDS_STAGE],
                                             int64_t m0, int64_t n0, int64_t kb, int nkf,
                                             Acc (&acc)[TM][TN], bool side) {
    const uint16_t* A = static_cast<const uint16_t*>(g.A);
    const uint16_t* B = static_cast<const uint16_t*>(g.B);
    dma_tile<BM>(A, g.lda, m0, kb, lds[0]);
    dma_tile<BN>(B, g.ldb, n0, kb, lds[0] + BM * CPR);
    if constexpr (kSideOut) {
      if (side) {
        if (late_wave())
          loop_side<true>(g, lds, m0, n0, kb, nkf, acc);
        else
          loop_side<false>(g, lds, m0, n0, kb, nkf, acc);
        __syncthreads();
        return;
      }
    }
    if (late_wave())
      loop_dma2<kLateStep>(g, lds, m0, n0, kb, nkf, acc);
    else
      loop_dma2<0>(g, lds, m0, n0, kb, nkf, acc);
    __syncthreads();
  }

  // One or both operands M/N-contiguous, interior block, whole K-tiles, two
  // stages: a K-contiguous operand is copied straight into the next stage
  // and an M/N-contiguous one staged through registers while the current
  // stage is multiplied. Loads for the next tile are issued before the
  // stage's first fragment reads (STEP 0) or before K step STEP.
  template <int STEP>
  static __device__ inline void loop_mixed(const GemmArgs& g, uint4 (*lds)[LDS_STAGE],
                                           int64_t m0, int64_t n0, int64_t kb, int nkf,
                                           Acc (&acc)[TM][TN]) {
    const uint16_t* A = static_cast<const uint16_t*>(g.A);
    const uint16_t* B = static_cast<const uint16_t*>(g.B);
    uint4 ra[A_K ? 1 : regs(BM, false)], rb[B_K ? 1 : regs(BN, false)];
    // all: every wave copies its share of a K-contiguous A (the first tile).
    // Otherwise, for 256 x 256 tiles with 8 waves, the early waves copy all of
    // A and the late waves only load their part of B, which keeps the late
    // waves' loads (the ones that bound the hand-off) short: grad_input at
    // 8192 x 4096 x 128256, 7.97 -> 7.85 ms.
    auto issue = [&](int64_t k0, uint4* st, bool all) {
      if constexpr (A_K && !B_K && kSplitCopies) {
        if (all)
          dma_tile<BM>(A, g.lda, m0, k0, st);
        else if constexpr (STEP == 0)
          dma_rows<BM / 32>(A, g.lda, m0, k0, st, 0, (threadIdx.x >> 6) % (NW / 2));
      } else if constexpr (A_K) {
        dma_tile<BM>(A, g.lda, m0, k0, st);
      } else {
        load_tile_fast<BM, false>(A, g.lda, m0, k0, ra);
      }
      if constexpr (B_K) dma_tile<BN>(B, g.ldb, n0, k0, st + BM * CPR);
      else load_tile_fast<BN, false>(B, g.ldb, n0, k0, rb);
    };
    auto finish = [&](uint4* st) {
      if constexpr (!A_K) store_tile<BM, false>(st, 0, ra);
      if constexpr (!B_K) store_tile<BN, false>(st, BM, rb);
    };
    issue(kb, lds[0], true);
    finish(lds[0]);
    wait_vmem_all();
    __syncthreads();
    for (int t = 0; t < nkf; ++t) {
      uint4* cur = lds[t & 1];
      uint4* nxt = lds[(t + 1) & 1];
      const bool more = t + 1 < nkf;
      const int64_t k0 = kb + static_cast<int64_t>(t + 1) * BK;
      if (STEP == 0 && more) issue(k0, nxt, false);
      compute_stage(cur, acc, [&](int ks) {
        if (STEP > 0 && more && ks == STEP) issue(k0, nxt, false);
      });
      if (more) finish(nxt);
      wait_vmem_all();
      __syncthreads();
    }
  }

  static __device__ inline void mainloop_mixed(const GemmArgs& g, uint4 (*lds)[LDS_STAGE],
                                               int64_t m0, int64_t n0, int64_t kb, int nkf,
                                               Acc (&acc)[TM][TN]) {
    if (late_wave())
      loop_mixed<kLateStep>(g, lds, m0, n0, kb, nkf, acc);
    else
      loop_mixed<0>(g, lds, m0, n0, kb, nkf, acc);
  }

  // Bounds-checked K-tiles [t0, t1) through registers (edge blocks, and the
  // partial last K-tile of interior blocks); two stages, one barrier per
  // K-tile; entered and left with every stage free.
  static __device__ inline void mainloop_checked(const GemmArgs& g, uint4 (*lds)[LDS_STAGE],
                                                 int64_t m0, int64_t n0, int64_t kb, int64_t ke,
                                                 int t0, int t1, Acc (&acc)[TM][TN]) {
    if (t0 >= t1) return;
    const uint16_t* A = static_cast<const uint16_t*>(g.A);
    const uint16_t* B = static_cast<const uint16_t*>(g.B);
    uint4 ra[regs(BM, A_K)], rb[regs(BN, B_K)];
    load_tile<BM, A_K>(A, g.lda, m0, g.M, kb + static_cast<int64_t>(t0) * BK, ke, ra);
    load_tile<BN, B_K>(B, g.ldb, n0, g.N, kb + static_cast<int64_t>(t0) * BK, ke, rb);
    store_tile<BM, A_K>(lds[0], 0, ra);
    store_tile<BN, B_K>(lds[0], BM, rb);
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
      uint4* cur = lds[(t - t0) & 1];
      uint4* nxt = lds[(t - t0 + 1) & 1];
      const bool more = t + 1 < t1;
      if (more) {
        const int64_t k0 = kb + static_cast<int64_t>(t + 1) * BK;
        load_tile<BM, A_K>(A, g.lda, m0, g.M, k0, ke, ra);
        load_tile<BN, B_K>(B, g.ldb, n0, g.N, k0, ke, rb);
      }
      compute_stage(cur, acc);
      if (more) {
        store_tile<BM, A_K>(nxt, 0, ra);
        store_tile<BN, B_K>(nxt, BM, rb);
      }
      __syncthreads();
    }
  }

  // bf16 store through LDS. The tile is written to LDS in 8-byte quads (a
  // lane's four consecutive columns in the transposed accumulator layout),
  // quad slot s of row r at s ^ (r % 16) so that the 16 rows a write
  // instruction covers land in distinct banks. Then each 32-lane
  // half-wave reads one 512-byte row back, a 16-byte chunk per lane from its
  // two quads' slots, and stores it to C with 16-byte writes. STATS: the same half-wave reduces the row's
  // rounded values to (max, sum 2^((z - max) k)) over the tile's valid
  // columns and writes them as the row's partial for N-tile tn.
  template <bool STATS>
  static __device__ inline void epilogue_staged(const GemmArgs& g, int64_t m0, int64_t n0, int tn,
                                                int lane, int wave_m, int wave_n,
                                                Acc (&acc)[TM][TN], uint4* lds) {
    constexpr int QPR = BN / 4;   // quads per row
    constexpr int CPR16 = BN / 8; // 16-byte chunks per row
    static_assert(CPR16 == 32, "one 32-lane half-wave per row");
    uint2* quads = reinterpret_cast<uint2*>(lds);
    __syncthreads();   // the stage buffers are free
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wave_m * WM + i * MS + lane % MS;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < NACC / 4; ++q) {
          const int col = wave_n * WN + j * MS + quad_col(lane, q);
          const int slot = (col >> 2) ^ (row & 15);
          quads[row * QPR + slot] =
              make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                         pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
        }
      }
    }
    __syncthreads();
    uint16_t* C = static_cast<uint16_t*>(g.C);
    const bool vec = (g.ldc & 7) == 0;
    const int c = threadIdx.x & 31;                 // 16-byte chunk of the row
    const int64_t n = n0 + 8 * c;
    // Interior tiles: straight-line code over kRowsAtOnce rows at a time, so
    // that the rows' LDS reads, stores and reduction chains overlap (the
    // general loop below, with its per-element bounds, is not unrolled).
    constexpr int kRowStep = NT / 32;
    constexpr int kRowsAtOnce = 4;
    if (m0 + BM <= g.M && n0 + BN <= g.N && vec) {
      static_assert(BM % (kRowStep * kRowsAtOnce) == 0, "whole groups of rows");
      for (int row0 = threadIdx.x >> 5; row0 < BM; row0 += kRowStep * kRowsAtOnce) {
        uint4 v[kRowsAtOnce];
#pragma unroll
        for (int u = 0; u < kRowsAtOnce; ++u) {
          // The chunk's two quads, each from its own slot (no swap to undo
          // where the row's XOR is odd).
          const int row = row0 + u * kRowStep;
          const int f = row & 15;
          const uint2 lo = quads[row * QPR + ((2 * c) ^ f)];
          const uint2 hi = quads[row * QPR + ((2 * c + 1) ^ f)];
          v[u] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
        // Non-temporal: the logits are read next by the loss passes, not by
        // this product (pass 2 0.71 -> 0.645 ms, logits -0.05 ms).
#pragma unroll
        for (int u = 0; u < kRowsAtOnce; ++u)
          st_stream(C + (m0 + row0 + u * kRowStep) * g.ldc + n, v[u]);
        if constexpr (STATS) {
          float z[kRowsAtOnce][8], mx[kRowsAtOnce], d[kRowsAtOnce];
#pragma unroll
          for (int u = 0; u < kRowsAtOnce; ++u) {
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) z[u][e] = __uint_as_float((w[e >> 1] >> (16 * (e & 1))) << 16);
            mx[u] = z[u][0];
#pragma unroll
            for (int e = 1; e < 8; ++e) mx[u] = fmaxf(mx[u], z[u][e]);
          }
#pragma unroll
          for (int u = 0; u < kRowsAtOnce; ++u) mx[u] = half_wave_max(mx[u]);
#pragma unroll
          for (int u = 0; u < kRowsAtOnce; ++u) {
            d[u] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d[u] += __builtin_amdgcn_exp2f((z[u][e] - mx[u]) * g.stat_k);
          }
#pragma unroll
          for (int u = 0; u < kRowsAtOnce; ++u) d[u] = half_wave_sum(d[u]);
          if (c == 0) {
#pragma unroll
            for (int u = 0; u < kRowsAtOnce; ++u)
              g.stat_part[(m0 + row0 + u * kRowStep) * g.stat_ld + tn] = make_float2(mx[u], d[u]);
          }
        }
      }
      return;
    }
    for (int row = threadIdx.x >> 5; row < BM; row += kRowStep) {
      const int f = row & 15;
      const uint2 lo = quads[row * QPR + ((2 * c) ^ f)];
      const uint2 hi = quads[row * QPR + ((2 * c + 1) ^ f)];
      const uint4 v = make_uint4(lo.x, lo.y, hi.x, hi.y);
      const int64_t m = m0 + row;
      if (m < g.M && n < g.N) {
        uint16_t* dst = C + m * g.ldc + n;
        if (vec && n + 8 <= g.N) {
          *reinterpret_cast<uint4*>(dst) = v;
        } else {
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
          for (int e = 0; e < 8; ++e)
            if (n + e < g.N) dst[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
        }
      }
      if constexpr (STATS) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          z[e] = n + e < g.N ? __uint_as_float((w[e >> 1] >> (16 * (e & 1))) << 16) : -INFINITY;
        // The row's maximum first (exact), then one exponential per element
        // against it; a tile row always holds at least one valid column.
        float mx = z[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[e]);
        mx = half_wave_max(mx);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d += __builtin_amdgcn_exp2f((z[e] - mx) * g.stat_k);
        d = half_wave_sum(d);
        if (c == 0 && m < g.M) g.stat_part[m * g.stat_ld + tn] = make_float2(mx, d);
      }
    }
  }

  // C = C + A B for bf16 or fp32 C, staged through LDS: the fp32 products of one
  // wave row (WM rows of the tile) at a time go to LDS (a lane's four
  // consecutive columns as one 16-byte write, chunk c of row r at
  // c ^ (r % 32)), then each 32-lane half-wave takes whole rows: it loads the
  // old values with 16-byte reads (all of its rows' loads issued first), adds
  // the fp32 products from LDS, rounds once and stores 16 bytes per lane.
  // Rows of one wave row's part (h) of the tile that a thread reads back:
  // pass p covers row h*WM + p*(NT/32) + thread/32, 8 columns at 8*(thread%32).
  static constexpr int kRowsPerPass = NT / 32;
  static constexpr int kPasses = WM / kRowsPerPass;

  // The read-add-write stages kSub parts of WM / kSub rows per wave row: the
  // 256-row tile (two wave rows) keeps half a wave row's products and four
  // passes of old values in flight at a time (fp32 C: 228 VGPRs instead of
  // 255 for whole 128-row wave rows; the same speed).
  static constexpr int kSub = WAVES_M > 1 ? 2 : 1;
  static constexpr int kPartRows = WM / kSub;
  static constexpr int kPartPasses = kPartRows / kRowsPerPass;
  static_assert(TM % kSub == 0 && kPartRows % kRowsPerPass == 0, "parts of whole MS-row tiles");

  // Old values of the part starting at tile row r0 (zero outside C), as
  // 16-byte vectors: one per pass for bf16, two for fp32.
  template <class Out, int NP>
  static __device__ inline void load_old(const GemmArgs& g, int64_t m0, int64_t n0, int r0,
                                         uint4 (&old)[NP][sizeof(Out) / 2]) {
    constexpr bool F32 = sizeof(Out) == 4;
    constexpr int V16 = sizeof(Out) / 2;
    const Out* C = static_cast<const Out*>(g.C);
    const bool vec = (g.ldc & (F32 ? 3 : 7)) == 0;
    const int64_t n = n0 + 8 * (threadIdx.x & 31);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int64_t m = m0 + r0 + p * kRowsPerPass + (threadIdx.x >> 5);
      uint32_t w[4 * V16];
#pragma unroll
      for (int k = 0; k < 4 * V16; ++k) w[k] = 0;
      if (m < g.M && n < g.N) {
        const Out* src = C + m * g.ldc + n;
        if (vec && n + 8 <= g.N) {
#pragma unroll
          for (int q = 0; q < V16; ++q) {
            const uint4 v = reinterpret_cast<const uint4*>(src)[q];
            w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
          }
        } else {
          for (int k = 0; k < 8; ++k) {
            if (n + k >= g.N) continue;
            if constexpr (F32) w[k] = __float_as_uint(src[k]);
            else w[k >> 1] |= static_cast<uint32_t>(src[k]) << (16 * (k & 1));
          }
        }
      }
#pragma unroll
      for (int q = 0; q < V16; ++q) old[p][q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
    }
  }

  // PRE: part 0's old values were loaded by the caller before the main loop
  // (one wave row only) and come in as pre.
  template <class Out, bool PRE>
  static __device__ inline void epilogue_accumulate_staged(const GemmArgs& g, int64_t m0,
                                                           int64_t n0, int lane, int wave_m,
                                                           int wave_n,
                                                           Acc (&acc)[TM][TN], uint4* lds,
                                                           const uint4 (*pre)[sizeof(Out) / 2]) {
    static_assert(BN == 256 && kPartRows * BN * 4 <= STAGES * LDS_STAGE * 16 &&
                      kPartRows % (NT / 32) == 0,
                  "one part of 1 KB fp32 rows fits in LDS, whole rows per half-wave");
    constexpr bool F32 = sizeof(Out) == 4;
    constexpr int V16 = sizeof(Out) / 2;         // 16-byte vectors of old values per lane and row
    constexpr int C16 = BN / 4;                  // fp32 16-byte chunks per row
    constexpr int ROWS_PER_PASS = kRowsPerPass;  // rows in flight per pass (one per half-wave)
    constexpr int PASSES = kPartPasses;
    constexpr int TMP = TM / kSub;               // MS-row tiles of a wave per part
    Out* C = static_cast<Out*>(g.C);
    const bool vec = (g.ldc & (F32 ? 3 : 7)) == 0;
    const int c8 = threadIdx.x & 31;             // 8-column group of the row
    const int64_t n = n0 + 8 * c8;
#pragma unroll
    for (int part = 0; part < WAVES_M * kSub; ++part) {
      const int h = part / kSub;                 // wave row
      const int sub = part % kSub;               // part of that wave row
      const int r_part = h * WM + sub * kPartRows;
      // Old values of this part's rows, loaded before the staging barrier
      // (or before the main loop).
      uint4 old[PASSES][V16];
      if constexpr (PRE) {
        static_assert(WAVES_M == 1 && kSub == 1, "prefetched old values cover the single part");
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
#pragma unroll
          for (int q = 0; q < V16; ++q) old[p][q] = pre[p][q];
      } else {
        load_old<Out, PASSES>(g, m0, n0, r_part, old);
      }
      __syncthreads();   // the stage buffers (or the previous part) are free
      if (wave_m == h) {
#pragma unroll
        for (int ii = 0; ii < TMP; ++ii) {
          const int i = sub * TMP + ii;
          const int row = ii * MS + lane % MS;  // within the part
#pragma unroll
          for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int q = 0; q < NACC / 4; ++q) {
              const int chunk = (wave_n * WN + j * MS + quad_col(lane, q)) >> 2;
              lds[row * C16 + (chunk ^ (row & 31))] =
                  make_uint4(__float_as_uint(acc[i][j][4 * q]), __float_as_uint(acc[i][j][4 * q + 1]),
                             __float_as_uint(acc[i][j][4 * q + 2]),
                             __float_as_uint(acc[i][j][4 * q + 3]));
            }
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int row = p * ROWS_PER_PASS + (threadIdx.x >> 5);
        const int64_t m = m0 + r_part + row;
        const uint4 a0 = lds[row * C16 + ((2 * c8) ^ (row & 31))];
        const uint4 a1 = lds[row * C16 + ((2 * c8 + 1) ^ (row & 31))];
        if (m >= g.M || n >= g.N) continue;
        const float add[8] = {__uint_as_float(a0.x), __uint_as_float(a0.y), __uint_as_float(a0.z),
                              __uint_as_float(a0.w), __uint_as_float(a1.x), __uint_as_float(a1.y),
                              __uint_as_float(a1.z), __uint_as_float(a1.w)};
        Out* dst = C + m * g.ldc + n;
        if constexpr (F32) {
          const uint32_t w[8] = {old[p][0].x, old[p][0].y, old[p][0].z, old[p][0].w,
                                 old[p][1].x, old[p][1].y, old[p][1].z, old[p][1].w};
          float out[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) out[e] = __uint_as_float(w[e]) + add[e];
          if (vec && n + 8 <= g.N) {
            reinterpret_cast<float4*>(dst)[0] = make_float4(out[0], out[1], out[2], out[3]);
            reinterpret_cast<float4*>(dst)[1] = make_float4(out[4], out[5], out[6], out[7]);
          } else {
            for (int e = 0; e < 8; ++e)
              if (n + e < g.N) dst[e] = out[e];
          }
        } else {
          const uint32_t w[4] = {old[p][0].x, old[p][0].y, old[p][0].z, old[p][0].w};
          uint32_t out[4];
#pragma unroll
          for (int d = 0; d < 4; ++d)
            out[d] = pack_bf16x2(bf16_lo(w[d]) + add[2 * d], bf16_hi(w[d]) + add[2 * d + 1]);
          if (vec && n + 8 <= g.N) {
            *reinterpret_cast<uint4*>(dst) = make_uint4(out[0], out[1], out[2], out[3]);
          } else {
            for (int e = 0; e < 8; ++e)
              if (n + e < g.N) dst[e] = static_cast<uint16_t>(out[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  }

  // Always inlined into the kernel: compiled as a call (the inliner's choice
  // for the largest variants), the body received its arguments through the
  // stack and read them from scratch memory inside the loops.
  static __device__ __attribute__((always_inline)) void run(const GemmArgs& g, int tiles_m, int tiles_n,
                                                           int group_m) {
    // The only __shared__ object of these kernels: with a second one the
    // compiler's LDS alias scopes make it wait for the direct copies in flight
    // before the main loop's fragment reads (measured: logits +0.7 ms).
    __shared__ uint4 lds[STAGES][LDS_STAGE];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wave_m = wave % WAVES_M;
    const int wave_n = wave / WAVES_M;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * BM;
    const int64_t n0 = static_cast<int64_t>(tn) * BN;
    const int split = blockIdx.y;
    const int64_t kb = static_cast<int64_t>(split) * g.k_per_split;
    const int64_t ke = min(g.K, kb + g.k_per_split);
    const int nk = static_cast<int>((ke - kb + BK - 1) / BK);

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < NACC; ++r) acc[i][j][r] = 0.f;

    // PRE_OLD (read-add-write with one wave row): the old values are loaded
    // before the main loop, in flight with the first tile's copies, so the
    // epilogue does not wait for them.
    using AccOut = typename std::conditional<EPI == kEpiAccumulateF32, float, uint16_t>::type;
    constexpr bool kPrefetchOld =
        PRE_OLD && (EPI == kEpiAccumulate || EPI == kEpiAccumulateF32) && WAVES_M == 1;
    uint4 pre_old[kPrefetchOld ? kPasses : 1][sizeof(AccOut) / 2];
    if constexpr (kPrefetchOld) load_old<AccOut, kPasses>(g, m0, n0, 0, pre_old);

    if (m0 + BM <= g.M && n0 + BN <= g.N) {
      const int nkf = static_cast<int>((ke - kb) / BK);   // whole K-tiles
      if (nkf > 0) {
        if constexpr (A_K && B_K)
          mainloop_dma(g, lds, m0, n0, kb, nkf, acc, SIDE && tm == side_tile_m(g, tn));
        else
          mainloop_mixed(g, lds, m0, n0, kb, nkf, acc);
      }
      mainloop_checked(g, lds, m0, n0, kb, ke, nkf, nk, acc);
    } else {
      mainloop_checked(g, lds, m0, n0, kb, ke, 0, nk, acc);
    }

    if constexpr (EPI == kEpiStore || EPI == kEpiStoreStats) {
      epilogue_staged<EPI == kEpiStoreStats>(g, m0, n0, tn, lane, wave_m, wave_n, acc, &lds[0][0]);
    } else if constexpr (EPI == kEpiAccumulate || EPI == kEpiAccumulateF32) {
      epilogue_accumulate_staged<AccOut, kPrefetchOld>(g, m0, n0, lane, wave_m, wave_n, acc,
                                                       &lds[0][0], pre_old);
    } else {
      // fp32 store (split-K partials, plane `split`), untransposed layout:
      // accumulator r of lane l holds row quad_col(l, r / 4) + r % 4, column
      // l % MS of its tile.
      static_assert(EPI == kEpiPartialF32, "epilogue");
      float* C = static_cast<float*>(g.C) + static_cast<int64_t>(split) * g.M * g.ldc;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int64_t n = n0 + wave_n * WN + j * MS + lane % MS;
          if (n >= g.N) continue;
#pragma unroll
          for (int r = 0; r < NACC; ++r) {
            const int64_t m = m0 + wave_m * WM + i * MS + quad_col(lane, r >> 2) + (r & 3);
            if (m < g.M) C[m * g.ldc + n] = acc[i][j][r];
          }
        }
      }
    }
  }
};

// Copy split of the 256 x 256 tiles' main loop per product (see kSplitCopies),
// measured inside the 8192 x 4096 x 128256 pass (each the best of 8 / 8 ..
// 14 / 2 copies per early / late wave): logits 10 / 6 (2 x 7.07 ms against
// 7.21 at 12 / 4), grad_input 9 / 7 (6.30 against 6.50), grad_W 9 / 7.
constexpr int kEarlyBLogits = 2;
constexpr int kEarlyBOther = 1;
constexpr int kEarlyBWgrad = 1;
template <int EPI>
constexpr int early_b() { return EPI == kEpiStoreStats ? kEarlyBLogits : kEarlyBOther; }

template <int BM, int BN, int BK, int STAGES, int WAVES_M, int WAVES_N, bool A_K, bool B_K,
          int EPI, bool PRE_OLD = false>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void gemm_bf16_kernel(GemmArgs g,
                                                                           int tiles_m,
                                                                           int tiles_n,
                                                                           int group_m) {
  GemmKernel<BM, BN, BK, STAGES, WAVES_M, WAVES_N, A_K, B_K, EPI, PRE_OLD, early_b<EPI>()>::run(
      g, tiles_m, tiles_n, group_m);
}

// The same code under a second symbol for the weight-gradient product, whose
// K-contiguous form (after the transposes) shares the logits product's layout.
template <int BM, int BN, int BK, int STAGES, int WAVES_M, int WAVES_N, bool A_K, bool B_K,
          int EPI, bool PRE_OLD = false>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void gemm_bf16_wgrad_kernel(GemmArgs g,
                                                                                 int tiles_m,
                                                                                 int tiles_n,
                                                                                 int group_m) {
  GemmKernel<BM, BN, BK, STAGES, WAVES_M, WAVES_N, A_K, B_K, EPI, PRE_OLD, kEarlyBWgrad>::run(
      g, tiles_m, tiles_n, group_m);
}

// The logits product that also writes B^T (GemmArgs::bt): a symbol of its own,
// so that no other launch carries the side output's code.
template <int BM, int BN, int BK, int STAGES, int WAVES_M, int WAVES_N, bool A_K, bool B_K,
          int EPI>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void gemm_bf16_side_kernel(GemmArgs g,
                                                                                int tiles_m,
                                                                                int tiles_n,
                                                                                int group_m) {
  GemmKernel<BM, BN, BK, STAGES, WAVES_M, WAVES_N, A_K, B_K, EPI, false, early_b<EPI>(), true>::run(
      g, tiles_m, tiles_n, group_m);
}

constexpr int kWavesM = 2;
constexpr int kWavesN = 4;

// K-tile and pipeline depth per layout (see the file comment).
template <bool A_K, bool B_K>
struct Pipe {
  static constexpr int BK = 64;
  static constexpr int STAGES = 2;
};

// Output tile (BM x 256) and wave grid (WM_ x WN_ waves) for one launch.
template <int BM, int WM_, int WN_, bool A_K, bool B_K, int EPI, bool PRE_OLD = false>
hipError_t launch_tiles(const GemmArgs& g, hipStream_t s) {
  const int64_t tiles_m = (g.M + BM - 1) / BM;
  const int64_t tiles_n = (g.N + kGemmBN - 1) / kGemmBN;
  const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n), static_cast<unsigned>(g.splitk));
  const dim3 block(WM_ * WN_ * 64);
  const int group_m = g.group_m > 0 ? static_cast<int>(std::min<int64_t>(g.group_m, tiles_m))
                                    : static_cast<int>(tiles_m);
  constexpr int BK = Pipe<A_K, B_K>::BK, ST = Pipe<A_K, B_K>::STAGES;
  if constexpr (A_K && B_K) {
    if (g.wgrad) {
      hipLaunchKernelGGL((gemm_bf16_wgrad_kernel<BM, kGemmBN, BK, ST, WM_, WN_, A_K, B_K, EPI, PRE_OLD>),
                         grid, block, 0, s, g, static_cast<int>(tiles_m),
                         static_cast<int>(tiles_n), group_m);
      return hipGetLastError();
    }
  }
  if constexpr (A_K && B_K && BM == kGemmBM && WM_ == kWavesM && WN_ == kWavesN &&
                (EPI == kEpiStore || EPI == kEpiStoreStats) && !PRE_OLD) {
    if (g.bt) {
      hipLaunchKernelGGL((gemm_bf16_side_kernel<BM, kGemmBN, BK, ST, WM_, WN_, A_K, B_K, EPI>), grid,
                         block, 0, s, g, static_cast<int>(tiles_m), static_cast<int>(tiles_n),
                         group_m);
      return hipGetLastError();
    }
  }
  if (g.bt) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, kGemmBN, BK, ST, WM_, WN_, A_K, B_K, EPI, PRE_OLD>), grid, block,
                     0, s, g, static_cast<int>(tiles_m), static_cast<int>(tiles_n), group_m);
  return hipGetLastError();
}

// Products with few rows (the logits and grad_input of small chunks) take
// 64-row tiles up to 64 rows and 128-row tiles up to 128, one row of eight
// wave tiles: a 256-row tile would spend most of its matrix-core work on rows
// that do not exist, and 64-row tiles let two workgroups share a CU. Between
// 65 and 128 rows one 128-row tile streams each weight panel once instead of
// twice (128 x 128256 x 4096 logits: 0.238 -> 0.221 ms).
constexpr int64_t kSkinnyMaxM = 128;

// The accumulating weight-gradient product of a chunk of at most kSkinnyMaxK
// rows is bound by each tile's serial load / multiply / read-add-write
// phases: 64-row tiles, two workgroups per CU, with the old values loaded
// before the (short) main loop so that they arrive with the first copies.
// From 256 rows up the 256-row tiles are faster (grad_W at 128256 x 4096 per
// pass of 8192 rows: 19.3 -> 18.0 ms at 256-row chunks, 11.3 -> 9.3 ms at
// 1024; at 1024 rows per pass: 3.24 against 3.63 ms at 128-row chunks,
// 5.77 against 6.57 at 64, 10.8 against 13.7 at 32).
constexpr int64_t kSkinnyMaxK = 128;

template <bool A_K, bool B_K, int EPI>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  if constexpr (EPI == kEpiStore || EPI == kEpiStoreStats || EPI == kEpiPartialF32) {
    if (g.M <= kSkinnyMaxM / 2 && !g.wgrad) return launch_tiles<64, 1, 8, A_K, B_K, EPI>(g, s);
    if (g.M <= kSkinnyMaxM && !g.wgrad) return launch_tiles<128, 1, 8, A_K, B_K, EPI>(g, s);
  }
  if constexpr (A_K && B_K && (EPI == kEpiAccumulate || EPI == kEpiAccumulateF32)) {
    if (g.wgrad && g.K <= kSkinnyMaxK) return launch_tiles<64, 1, 8, A_K, B_K, EPI, true>(g, s);
  }
  return launch_tiles<kGemmBM, kWavesM, kWavesN, A_K, B_K, EPI>(g, s);
}

template <bool A_K, bool B_K>
hipError_t launch_layout(const GemmArgs& g, hipStream_t s) {
  switch (g.epilogue) {
    case kEpiStore: return launch_cfg<A_K, B_K, kEpiStore>(g, s);
    case kEpiAccumulate: return launch_cfg<A_K, B_K, kEpiAccumulate>(g, s);
    case kEpiPartialF32: return launch_cfg<A_K, B_K, kEpiPartialF32>(g, s);
    case kEpiStoreStats:
      // Only the logits product reduces row statistics.
      if constexpr (A_K && B_K) return launch_cfg<A_K, B_K, kEpiStoreStats>(g, s);
      return hipErrorInvalidValue;
    case kEpiAccumulateF32:
      // Only the weight-gradient product accumulates into an fp32 C.
      if constexpr (A_K && B_K) return launch_cfg<A_K, B_K, kEpiAccumulateF32>(g, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  // B^T is written only by the 256 x 256 tiles' whole-K-tile loop with a
  // store epilogue: refuse every other launch rather than leave it unwritten.
  if (g.bt) {
    const bool ok = g.a_kcontig && g.b_kcontig && !g.wgrad && g.splitk == 1 &&
                    (g.epilogue == kEpiStore || g.epilogue == kEpiStoreStats) &&
                    g.M >= kGemmBM && g.N % kGemmBN == 0 &&
                    g.K % Pipe<true, true>::BK == 0 && g.ldbt >= g.N;
    if (!ok) return hipErrorInvalidValue;
  }
  // The two layouts the pass uses: both operands K-contiguous (logits, and
  // the weight gradient after its transposes), and B N-contiguous
  // (grad_input's weight operand).
  if (g.a_kcontig && g.b_kcontig) return launch_layout<true, true>(g, s);
  if (g.a_kcontig && !g.b_kcontig) return launch_layout<true, false>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace fljsd
