// Chunk, slice, split-K and workspace planning (host arithmetic only).
//
// Chunking follows the pages' per-chunk memory model (Liger-Kernel PR #1352,
// Details, memory table): one chunk of C rows holds both logits tensors,
// 2 * C * V * s bytes, and only the per-row loss scales with BT. The policy
// replaces the cdiv(V, H) heuristic that the same page (Open question 4)
// calls mis-tuned for JSD: it takes the largest chunk that fits.
#include "plan.h"

#include <algorithm>

namespace fljsd {

SlicePlan plan_slices(int64_t rows, int64_t V) {
  SlicePlan sp;
  int64_t S = 1;
  if (rows < kJsdTargetBlocks) {
    S = cdiv(kJsdTargetBlocks, rows);
    S = std::min<int64_t>(S, std::max<int64_t>(1, V / kJsdMinSlice));
    S = std::min<int64_t>(S, 64);
  }
  sp.slice_w = round_up(cdiv(V, S), kJsdVec);
  sp.S = static_cast<int>(cdiv(V, sp.slice_w));
  return sp;
}

void plan_splitk(int64_t M, int64_t N, int64_t K, int* splitk, int64_t* k_per_split) {
  const int64_t tiles = cdiv(M, kGemmBM) * cdiv(N, kGemmBN);
  // Products of at most 64 rows run 64-row tiles, two workgroups per CU.
  const int64_t target = M <= 64 ? 2 * kGemmTargetBlocks : kGemmTargetBlocks;
  int64_t s = 1;
  if (tiles < target * 3 / 4) {
    s = cdiv(target, tiles);
    // Keep at least four K-tiles per split.
    s = std::min<int64_t>(s, std::max<int64_t>(1, K / (4 * kGemmBK)));
  }
  int64_t kps = round_up(cdiv(K, s), kGemmBK);
  s = cdiv(K, kps);
  *splitk = static_cast<int>(s);
  *k_per_split = kps;
}

ChunkPlan plan_chunks(int64_t BT, int64_t H_s, int64_t H_t, int64_t V, int dtype,
                      int64_t num_chunks) {
  ChunkPlan p;
  p.BT = BT;
  p.H_s = H_s;
  p.H_t = H_t;
  p.V = V;
  p.dtype = dtype;
  p.C = cdiv(BT, num_chunks);
  p.n_chunks = cdiv(BT, p.C);
  p.ldz = round_up(V, kJsdVec);
  p.slices = plan_slices(p.C, V);
  const int64_t es = dtype_size(dtype);
  if (dtype == 1) {
    plan_splitk(p.C, H_s, V, &p.splitk, &p.k_per_split);
  } else {
    p.splitk = 1;
    p.k_per_split = V;
  }
  p.transposed_grad_w = dtype == 1;
  p.ldt = round_up(p.C, kJsdVec);
  const int64_t zt_elems = p.C * p.ldz;
  size_t off = 0;
  p.off_zs = off;
  off = align256(off + static_cast<size_t>(p.C * p.ldz * es));
  p.off_zt = off;
  off = align256(off + static_cast<size_t>(zt_elems * es));
  p.off_row_loss = off;
  off = align256(off + static_cast<size_t>(BT) * 4);
  p.off_stats = off;
  off = align256(off + static_cast<size_t>(p.C * p.slices.S) * 16);
  p.off_lg = off;
  off = align256(off + static_cast<size_t>(p.C * p.slices.S) * 8);
  p.off_peak = off;
  off = align256(off + static_cast<size_t>(p.C * p.slices.S) * 16);
  p.off_ref = off;
  off = align256(off + static_cast<size_t>(p.C * p.slices.S) * 4);
  p.off_partial = off;
  if (p.splitk > 1) off = align256(off + static_cast<size_t>(p.splitk) * p.C * H_s * 4);
  p.off_xt = off;
  if (p.transposed_grad_w) off = align256(off + static_cast<size_t>(H_s * p.ldt * es));
  p.off_dzt = off;
  if (p.transposed_grad_w) off = align256(off + static_cast<size_t>(V * p.ldt * es));
  p.gemm_stats = dtype == 1;
  p.stat_tiles = cdiv(V, kGemmBN);
  p.off_spart = off;
  if (p.gemm_stats) off = align256(off + static_cast<size_t>(2 * p.C * p.stat_tiles) * 8);
  p.total = off;
  return p;
}

JsdPlan plan_jsd(int64_t BT, int64_t V) {
  JsdPlan p;
  p.slices = plan_slices(BT, V);
  size_t off = 0;
  p.off_row_loss = off;
  off = align256(off + static_cast<size_t>(BT) * 4);
  p.off_stats = off;
  off = align256(off + static_cast<size_t>(BT * p.slices.S) * 16);
  p.off_lg = off;
  off = align256(off + static_cast<size_t>(BT * p.slices.S) * 8);
  p.off_peak = off;
  off = align256(off + static_cast<size_t>(BT * p.slices.S) * 16);
  p.off_ref = off;
  off = align256(off + static_cast<size_t>(BT * p.slices.S) * 4);
  p.total = off;
  return p;
}

CePlan plan_ce_chunks(int64_t BT, int64_t H, int64_t V, int dtype, int64_t num_chunks) {
  CePlan p;
  p.C = cdiv(BT, num_chunks);
  p.n_chunks = cdiv(BT, p.C);
  p.ldz = round_up(V, kJsdVec);
  p.ldt = round_up(p.C, kJsdVec);
  p.slices = plan_slices(p.C, V);
  const int64_t es = dtype_size(dtype);
  if (dtype == 1) {
    plan_splitk(p.C, H, V, &p.splitk, &p.k_per_split);
  } else {
    p.splitk = 1;
    p.k_per_split = V;
  }
  p.transposed_grad_w = dtype == 1;
  size_t off = 0;
  p.off_z = off;
  off = align256(off + static_cast<size_t>(p.C * p.ldz * es));
  p.off_zt = off;
  if (p.transposed_grad_w) off = align256(off + static_cast<size_t>(V * p.ldt * es));
  p.off_xt = off;
  if (p.transposed_grad_w) off = align256(off + static_cast<size_t>(H * p.ldt * es));
  p.off_row_loss = off;
  off = align256(off + static_cast<size_t>(BT) * 4);
  p.off_stats = off;
  off = align256(off + static_cast<size_t>(p.C * p.slices.S) * 16);
  p.off_zy = off;
  off = align256(off + static_cast<size_t>(p.C) * 4);
  p.off_scale = off;
  off = align256(off + 16);
  p.off_partial = off;
  if (p.splitk > 1) off = align256(off + static_cast<size_t>(p.splitk) * p.C * H * 4);
  p.total = off;
  return p;
}

int64_t policy_num_chunks_ce(int64_t BT, int64_t H, int64_t V, int dtype, size_t budget) {
  int64_t nc = 1;
  while (nc <= BT) {
    const CePlan p = plan_ce_chunks(BT, H, V, dtype, nc);
    if (p.total <= budget) return nc;
    if (p.C == 1) break;
    nc = cdiv(BT, p.C - 1);
  }
  return 0;
}

int64_t policy_num_chunks(int64_t BT, int64_t H_s, int64_t H_t, int64_t V, int dtype,
                          size_t budget) {
  // Distinct chunk sizes only: C = ceil(BT / nc) changes at most 2*sqrt(BT) times.
  int64_t nc = 1;
  while (nc <= BT) {
    ChunkPlan p = plan_chunks(BT, H_s, H_t, V, dtype, nc);
    if (p.total <= budget) return nc;
    // Next nc that gives a smaller chunk.
    const int64_t C = p.C;
    if (C == 1) break;
    nc = cdiv(BT, C - 1);
  }
  return 0;
}

}  // namespace fljsd
