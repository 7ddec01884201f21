// Host-side planning for the fused-linear JSD pass: chunk geometry, the
// V-slicing of the loss kernels, the split-K factor of the grad_input GEMM and
// the workspace layout. Pure integer arithmetic; no HIP calls.
#pragma once

#include <cstddef>
#include <cstdint>
#include <climits>

namespace fljsd {

// Tile shape of the bf16 MFMA GEMMs (rows x columns of one workgroup's output).
constexpr int kGemmBM = 256;
constexpr int kGemmBN = 256;
constexpr int kGemmBK = 64;
// Writing W_s^T costs the first logits product a fixed ~0.4 ms at V = 128256,
// H_s = 4096, and each grad_input row gains ~0.08 us: measured at H_s = 4096
// (one chunk) +0.13 ms at 2048 rows, +0.1 at 4096, -0.2 at 6144, -0.3 at
// 8192, -0.9 at 16384; neutral at 256-row chunks, where every workgroup of
// the first product writes.
constexpr int64_t kWtMinRows = 4096;
constexpr int64_t kWtMinChunk = 512;
// Tile shape of the fp32 GEMMs.
constexpr int kGemmF32BM = 64;
constexpr int kGemmF32BN = 64;

// The loss kernels' workgroup: 256 threads, 8 elements per thread per step.
constexpr int kJsdThreads = 256;
constexpr int kJsdVec = 8;
// Aim for at least this many workgroups per loss-kernel launch.
constexpr int64_t kJsdTargetBlocks = 2048;
// Minimum elements of one row a loss workgroup covers when a row is split.
constexpr int64_t kJsdMinSlice = 4096;
// Aim for at least this many workgroups in the grad_input GEMM.
constexpr int64_t kGemmTargetBlocks = 256;

// Largest BT, H or V the planner takes (2^40): with every size at most this,
// no intermediate of the plan arithmetic overflows int64; workspace totals
// are summed with saturation at kSizeOverflow.
constexpr int64_t kMaxPlanDim = int64_t(1) << 40;
constexpr size_t kSizeOverflow = SIZE_MAX;

// a / b rounded up, for a >= 0, b > 0 (no a + b - 1 that could overflow).
inline int64_t cdiv(int64_t a, int64_t b) { return a / b + (a % b != 0 ? 1 : 0); }
inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Workspace layout: regions of n * m * es bytes, each starting 256-byte
// aligned; the total saturates at kSizeOverflow instead of wrapping.
struct Layout {
  size_t off = 0;
  size_t take(int64_t n, int64_t m, int64_t es) {
    const size_t at = off;
    size_t bytes = 0;
    if (off == kSizeOverflow || __builtin_mul_overflow(static_cast<size_t>(n), static_cast<size_t>(m), &bytes) ||
        __builtin_mul_overflow(bytes, static_cast<size_t>(es), &bytes) ||
        __builtin_add_overflow(off, bytes, &off) || off > kSizeOverflow - 255) {
      off = kSizeOverflow;
      return kSizeOverflow;
    }
    off = (off + 255) & ~size_t(255);
    return at;
  }
};

inline int dtype_size(int dtype) { return dtype == 0 ? 4 : 2; }
// Elements per 16-byte vector for the dtype.
inline int dtype_vec(int dtype) { return dtype == 0 ? 4 : 8; }

// Column span of one workgroup of the bf16 gradient pass (64-row x 64-column
// tiles): as many 64-column tiles as keep about kGradTargetBlocks workgroups in
// the launch, at most kGradTileColsMax columns; nblk column blocks per row.
constexpr int64_t kGradTileColsMax = 1024;
constexpr int64_t kGradTargetBlocks = 2048;
inline void grad_t_geometry(int64_t rows, int64_t V, int64_t* span, int64_t* nblk) {
  const int64_t row_blocks = cdiv(rows, 64);
  const int64_t tiles = cdiv(V, 64);
  int64_t work = 0;
  if (__builtin_mul_overflow(tiles, row_blocks, &work)) work = INT64_MAX;
  int64_t per = cdiv(work, kGradTargetBlocks);
  per = per < 1 ? 1 : (per > kGradTileColsMax / 64 ? kGradTileColsMax / 64 : per);
  *span = per * 64;
  *nblk = cdiv(V, *span);
}

struct SlicePlan {
  int S = 1;             // slices per row
  int64_t slice_w = 0;   // elements per slice, a multiple of kJsdVec
};

// Slices per row for `rows` rows of V columns: enough workgroups to fill the
// chip when there are few rows, never slices narrower than kJsdMinSlice.
SlicePlan plan_slices(int64_t rows, int64_t V);

struct ChunkPlan {
  int64_t BT = 0, H_s = 0, H_t = 0, V = 0;
  int dtype = 0;
  int64_t C = 0;          // rows per chunk
  int64_t n_chunks = 0;   // chunks actually run: ceil(BT / C)
  int64_t ldz = 0;        // row stride (elements) of the logits chunk buffers
  // bf16: dZ^T [V, ldt] and X_s^T [H_s, ldt] have regions of their own, so
  // grad_W = dZ^T X_s reads both operands with K (rows) fastest. dZ^T cannot
  // share the teacher-logits buffer: pass 3 writes it while it still reads Z_t.
  bool transposed_grad_w = false;
  int64_t ldt = 0;        // row stride of the transposed operands: C rounded up to 8
  // bf16: the logits GEMMs reduce each row's statistics per N-tile into
  // [C, stat_tiles] float2 partials (student, then teacher), replacing pass 1's
  // read of both logits rows.
  bool gemm_stats = false;
  int64_t stat_tiles = 0;
  SlicePlan slices;       // for C rows
  int splitk = 1;         // split-K factor of grad_input = dZ W_s
  int64_t k_per_split = 0;
  // bf16 with V a multiple of the GEMM N tile, H_s of its K tile, more than
  // kWtMinRows rows in all and chunks of at least kWtMinChunk rows: W_s^T
  // [H_s, ldz] has a region of its own. The first chunk's student logits
  // product writes it from the W_s tiles it holds in LDS, and grad_input =
  // dZ W_s then reads both operands K-contiguous.
  bool w_transposed = false;
  // Workspace layout, byte offsets from the workspace base. total_min leaves
  // out the W_s^T region (the last one): a workspace of at least total_min but
  // under total bytes runs without it.
  size_t off_zs = 0, off_zt = 0, off_row_loss = 0, off_stats = 0, off_lg = 0, off_peak = 0,
         off_ref = 0, off_lpart = 0, off_partial = 0, off_xt = 0, off_spart = 0, off_dzt = 0,
         off_wst = 0, total_min = 0, total = 0;
};

// Turns the W_s^T region off: grad_input reads W_s as given.
void drop_w_transposed(ChunkPlan* p);

// Chunk plan for num_chunks >= 1 (C = ceil(BT / num_chunks)).
ChunkPlan plan_chunks(int64_t BT, int64_t H_s, int64_t H_t, int64_t V, int dtype,
                      int64_t num_chunks);

// Split-K choice for an M x N output with K-dimension K on the bf16 GEMM.
void plan_splitk(int64_t M, int64_t N, int64_t K, int* splitk, int64_t* k_per_split);

struct JsdPlan {
  SlicePlan slices;
  size_t off_row_loss = 0, off_stats = 0, off_lg = 0, off_peak = 0, off_ref = 0, total = 0;
};

JsdPlan plan_jsd(int64_t BT, int64_t V);

// Smallest num_chunks whose workspace (less the optional W_s^T region) fits
// the budget; 0 if none does.
int64_t policy_num_chunks(int64_t BT, int64_t H_s, int64_t H_t, int64_t V, int dtype,
                          size_t budget);

// Fused-linear cross-entropy: one logits chunk, the same GEMM planning.
struct CePlan {
  int64_t C = 0, n_chunks = 0, ldz = 0, ldt = 0;
  SlicePlan slices;
  int splitk = 1;
  int64_t k_per_split = 0;
  bool transposed_grad_w = false;
  bool w_transposed = false;   // W^T [H, ldz] for grad_input, as in ChunkPlan
  size_t off_z = 0, off_zt = 0, off_xt = 0, off_row_loss = 0, off_stats = 0, off_zy = 0,
         off_scale = 0, off_partial = 0, off_wt = 0, total_min = 0, total = 0;
};
void drop_w_transposed(CePlan* p);

CePlan plan_ce_chunks(int64_t BT, int64_t H, int64_t V, int dtype, int64_t num_chunks);
// Smallest num_chunks whose workspace (less the optional W^T region) fits.
int64_t policy_num_chunks_ce(int64_t BT, int64_t H, int64_t V, int dtype, size_t budget);

}  // namespace fljsd
