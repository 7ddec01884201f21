// Chunk, slice, split-K and workspace planning (host arithmetic only).
//
// Chunking follows the pages' per-chunk memory model (Liger-Kernel PR #1352,
// Details, memory table): one chunk of C rows holds both logits tensors,
// 2 * C * V * s bytes, and only the per-row loss scales with BT. For bf16 with
// a weight gradient a third logits-sized region holds dZ^T (written by pass 3,
// read by the weight-gradient product), 3 * C * V * s in all, plus X_s^T and
// the per-row statistics, and (shapes that tile evenly) W_s^T, V * H_s * s,
// for the grad_input product. The policy replaces the cdiv(V, H) heuristic that
// the same page (Open question 4) calls mis-tuned for JSD: it takes the
// largest chunk that fits.
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
  // Output tiles, capped: only whether they fill the chip matters.
  const int64_t tm = cdiv(M, kGemmBM), tn = cdiv(N, kGemmBN);
  const int64_t tiles = tm > (int64_t(1) << 20) || tn > (int64_t(1) << 20) ? (int64_t(1) << 40) : tm * tn;
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
  const int64_t rs = p.C * p.slices.S;   // row-slice pairs of one chunk
  Layout L;
  p.off_zs = L.take(p.C, p.ldz, es);
  p.off_zt = L.take(p.C, p.ldz, es);
  p.off_row_loss = L.take(BT, 1, 4);
  p.off_stats = L.take(rs, 1, 16);
  p.off_lg = L.take(rs, 1, 8);
  p.off_peak = L.take(rs, 1, 16);
  p.off_ref = L.take(rs, 1, 4);
  {
    // bf16 with a weight gradient: pass 3's per-row loss partials, sized for
    // both chunk lengths the plan runs (C, and the last chunk's).
    int64_t span = 0, nblk = 0, nblk_last = 0;
    const int64_t last = BT - (p.n_chunks - 1) * p.C;
    grad_t_geometry(p.C, V, &span, &nblk);
    grad_t_geometry(last, V, &span, &nblk_last);
    int64_t n = 0, n_last = 0;
    if (__builtin_mul_overflow(nblk, p.C, &n)) n = INT64_MAX;
    if (__builtin_mul_overflow(nblk_last, last, &n_last)) n_last = INT64_MAX;
    p.off_lpart = L.take(dtype == 1 ? std::max(n, n_last) : 0, 1, 4);
  }
  p.off_partial = L.take(p.splitk > 1 ? p.splitk * p.C : 0, H_s, 4);
  p.off_xt = L.take(p.transposed_grad_w ? H_s : 0, p.ldt, es);
  p.off_dzt = L.take(p.transposed_grad_w ? V : 0, p.ldt, es);
  p.gemm_stats = dtype == 1;
  p.stat_tiles = cdiv(V, kGemmBN);
  p.off_spart = L.take(p.gemm_stats ? 2 * p.C : 0, p.stat_tiles, 8);
  p.total_min = L.off;
  // W_s^T last, so that a workspace of total_min bytes holds everything else.
  p.w_transposed = dtype == 1 && V % kGemmBN == 0 && H_s % kGemmBK == 0 &&
                   BT > kWtMinRows && p.C >= kWtMinChunk;
  p.off_wst = L.take(p.w_transposed ? H_s : 0, p.ldz, es);
  p.total = L.off;
  if (p.total == kSizeOverflow) drop_w_transposed(&p);
  return p;
}

void drop_w_transposed(ChunkPlan* p) {
  p->w_transposed = false;
  p->off_wst = 0;
  p->total = p->total_min;
}

JsdPlan plan_jsd(int64_t BT, int64_t V) {
  JsdPlan p;
  p.slices = plan_slices(BT, V);
  const int64_t rs = BT * p.slices.S;
  Layout L;
  p.off_row_loss = L.take(BT, 1, 4);
  p.off_stats = L.take(rs, 1, 16);
  p.off_lg = L.take(rs, 1, 8);
  p.off_peak = L.take(rs, 1, 16);
  p.off_ref = L.take(rs, 1, 4);
  p.total = L.off;
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
  Layout L;
  p.off_z = L.take(p.C, p.ldz, es);
  p.off_zt = L.take(p.transposed_grad_w ? V : 0, p.ldt, es);
  p.off_xt = L.take(p.transposed_grad_w ? H : 0, p.ldt, es);
  p.off_row_loss = L.take(BT, 1, 4);
  p.off_stats = L.take(p.C * p.slices.S, 1, 16);
  p.off_zy = L.take(p.C, 1, 4);
  p.off_scale = L.take(16, 1, 1);
  p.off_partial = L.take(p.splitk > 1 ? p.splitk * p.C : 0, H, 4);
  p.total_min = L.off;
  // W^T last (the same rule and reason as the JSD pass's W_s^T region).
  p.w_transposed = dtype == 1 && V % kGemmBN == 0 && H % kGemmBK == 0 && BT > kWtMinRows &&
                   p.C >= kWtMinChunk;
  p.off_wt = L.take(p.w_transposed ? H : 0, p.ldz, es);
  p.total = L.off;
  if (p.total == kSizeOverflow) drop_w_transposed(&p);
  return p;
}

void drop_w_transposed(CePlan* p) {
  p->w_transposed = false;
  p->off_wt = 0;
  p->total = p->total_min;
}

int64_t policy_num_chunks_ce(int64_t BT, int64_t H, int64_t V, int dtype, size_t budget) {
  int64_t nc = 1;
  while (nc <= BT) {
    const CePlan p = plan_ce_chunks(BT, H, V, dtype, nc);
    if (p.total_min != kSizeOverflow && p.total_min <= budget) return nc;
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
    // The optional W_s^T region never costs a chunk.
    if (p.total_min != kSizeOverflow && p.total_min <= budget) return nc;
    // Next nc that gives a smaller chunk.
    const int64_t C = p.C;
    if (C == 1) break;
    nc = cdiv(BT, C - 1);
  }
  return 0;
}

}  // namespace fljsd
