// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fljsd {

// Which branch of the divergence a launch evaluates (PR #1352, Testing Done:
// beta 0.0 is forward KL, 1.0 reverse KL, anything between generalized).
enum JsdMode : int { kModeGeneralized = 0, kModeForwardKL = 1, kModeReverseKL = 2 };

struct JsdArgs {
  const void* zs = nullptr;     // student logits [rows, ld]
  const void* zt = nullptr;     // teacher logits [rows, ld]
  void* grad = nullptr;         // dZ destination [rows, ld]; may equal zs
  int64_t ld = 0;
  bool vec_ok = true;           // ld is a whole number of 16-byte vectors
  int64_t rows = 0;
  int64_t V = 0;
  int64_t slice_w = 0;
  int S = 1;
  float k2 = 0.f;               // log2(e) / T: base-2 scaled logit factor
  float beta = 0.f;
  float grad_scale = 0.f;       // reduction scale / T
  int mode = kModeGeneralized;
  float4* stats = nullptr;      // [rows * S] partial (m_s, d_s, m_t, d_t), base 2
  float2* lg = nullptr;         // [rows * S] partial (loss, dX_sum)
  // [rows * S] fp32 inputs only: partial (Q_rest, P_rest, g_rest, n) over the
  // row's elements below / at the student's maximum logit (see jsd_grad_kernel)
  float4* peak = nullptr;
  // [rows * S] fp32 inputs only: pass 1's teacher logit at the student's
  // maximum logit (the largest, if the maximum is tied), the reference element
  // of the gradient terms (see jsd_loss_kernel)
  float* ref = nullptr;
  float* lpart = nullptr;       // [column blocks][rows] bf16 pass 3's loss partials
  float* row_loss = nullptr;    // [rows] per-row loss out
  float row_scale = 1.f;        // multiplies the per-row losses (T^2 when asked)
};

// The one-pass losses over given distributions (log-probability JSD, TVD).
struct ElemArgs {
  const void* a = nullptr;      // student log-probabilities, or p   [rows, ld]
  const void* b = nullptr;      // teacher log-probabilities, or q   [rows, ld]
  void* grad = nullptr;         // d loss / d a [rows, ld], or null; may equal a
  float* elem_loss = nullptr;   // TVD elementwise losses [rows, V] (reduction none)
  int64_t ld = 0;
  bool vec_ok = true;
  int64_t rows = 0;
  int64_t V = 0;
  int64_t slice_w = 0;
  int S = 1;
  float beta = 0.f;
  float grad_scale = 0.f;       // reduction scale
  int mode = kModeGeneralized;
  float2* lg = nullptr;         // [rows * S] partial loss sums (.x)
};
hipError_t launch_logprob_jsd(const ElemArgs& a, int dtype, hipStream_t s);
hipError_t launch_tvd(const ElemArgs& a, int dtype, hipStream_t s);

// Cross-entropy over a logits chunk with hard labels.
struct CeArgs {
  const void* z = nullptr;        // logits [rows, ld]
  void* grad = nullptr;           // dZ [rows, ld]; may equal z
  int64_t ld = 0;
  bool vec_ok = true;
  int64_t rows = 0;
  int64_t V = 0;
  int64_t slice_w = 0;
  int S = 1;
  const int64_t* labels = nullptr;  // [rows]
  int64_t ignore_index = -100;
  float eps = 0.f;                // label smoothing
  float4* stats = nullptr;        // [rows * S] partial (m, d, sum z, -), d base 2
  float* zy = nullptr;            // [rows] logit of the label
  const float* scale = nullptr;   // device: [0] gradient scale, [1] loss scale
  float* row_loss = nullptr;      // [rows]
};
// scale[0], scale[1] from the labels of all BT rows (reduction as fljsd_reduction).
hipError_t launch_ce_scale(const int64_t* labels, int64_t BT, int64_t V, int64_t ignore_index,
                           int reduction, float* scale, hipStream_t s);
hipError_t launch_ce_stats(const CeArgs& a, int dtype, hipStream_t s);
hipError_t launch_ce_grad(const CeArgs& a, int dtype, bool write_grad, hipStream_t s);
// bf16 pass 2 that also writes dZ^T [V, ldt] (the weight-gradient operand).
hipError_t launch_ce_grad_transposed(const CeArgs& a, void* dzt, int64_t ldt, hipStream_t s);
// loss[0] = scale[1] * sum(row_loss[0..n)), deterministic order.
hipError_t launch_loss_reduce_dev(const float* row_loss, int64_t n, const float* scale,
                                  float* loss, hipStream_t s);

// Loss passes. dtype: 0 = fp32, 1 = bf16.
hipError_t launch_jsd_stats(const JsdArgs& a, int dtype, hipStream_t s);
hipError_t launch_jsd_loss(const JsdArgs& a, int dtype, hipStream_t s);
hipError_t launch_jsd_grad(const JsdArgs& a, int dtype, hipStream_t s);
// Pass 3 for bf16 that also writes dZ^T [V, ldt] (the weight-gradient operand).
// loss_in_pass3 (generalized and forward KL): pass 3 also sums the loss terms
// into a.lpart (after launch_jsd_gsum, or no pass 2 at all for the forward
// KL); launch_jsd_row_loss_merge then writes the row losses.
hipError_t launch_jsd_grad_transposed(const JsdArgs& a, void* dzt, int64_t ldt, bool loss_in_pass3,
                                      hipStream_t s);
hipError_t launch_jsd_gsum(const JsdArgs& a, hipStream_t s);
hipError_t launch_jsd_row_loss_merge(const JsdArgs& a, hipStream_t s);
// Pass 1 from the logits GEMMs' row-statistic partials [rows, tiles] (student,
// teacher): writes the row statistics the loss passes read.
hipError_t launch_jsd_stats_merge(const JsdArgs& a, const float2* part_s, const float2* part_t,
                                  int64_t tiles, hipStream_t s);
// Per-row loss only (no gradient written): merges the pass-2 partials.
hipError_t launch_jsd_row_loss(const JsdArgs& a, hipStream_t s);
// loss[0] = scale * sum(row_loss[0..n)), deterministic order.
hipError_t launch_loss_reduce(const float* row_loss, int64_t n, float scale, float* loss,
                              hipStream_t s);
// out[m, n] (dtype, ld ldo) = sum over splits of part[split][m][n] (fp32, ld N).
hipError_t launch_splitk_reduce(const float* part, int splits, int64_t M, int64_t N,
                                void* out, int64_t ldo, int dtype, hipStream_t s);

// GEMM operand layouts. An operand is "K-contiguous" when its reduction index
// is the fastest-varying one in memory.
enum GemmEpilogue : int {
  kEpiStore = 0,        // C = A B, rounded once to the dtype
  kEpiAccumulate = 1,   // C = C + A B, added in fp32 and rounded once
  kEpiPartialF32 = 2,   // fp32 partial sum of one K-split at C + split * M * ldc
                        // (with one split: C = A B stored in fp32)
  kEpiAccumulateF32 = 3,  // fp32 C = C + A B, no rounding (bf16 operands)
  kEpiStoreStats = 4,     // kEpiStore, plus each row's (max, sum 2^((z-max) k)) over
                          // the tile's columns of the rounded values, per N-tile
};

struct GemmArgs {
  const void* A = nullptr;
  const void* B = nullptr;
  void* C = nullptr;
  int64_t M = 0, N = 0, K = 0;
  int64_t lda = 0, ldb = 0, ldc = 0;
  bool a_kcontig = true;   // A(m,k) = A[m*lda + k]  else  A[k*lda + m]
  bool b_kcontig = true;   // B(n,k) = B[n*ldb + k]  else  B[k*ldb + n]
  int epilogue = kEpiStore;
  int splitk = 1;
  int64_t k_per_split = 0; // multiple of the K tile when splitk > 1
  int group_m = 0;         // M-tiles per tile group in the launch order (0: all)
  bool wgrad = false;      // the weight-gradient product (its own kernel symbol, so
                           // profiles tell it from the logits product)
  // kEpiStoreStats: partial row statistics [M, stat_ld] float2 (max in logit
  // units, denominator in base 2 with scale stat_k), one per N-tile.
  float2* stat_part = nullptr;
  int64_t stat_ld = 0;
  float stat_k = 0.f;
  // Both operands K-contiguous, bf16: when set, one workgroup per N-tile
  // (its M-tile rotating with the N-tile, so the writers spread over the
  // XCDs) also writes B transposed, bt[k * ldbt + n] = B(n, k), from the B
  // tiles it holds in LDS. Needs every such block interior: N a multiple of
  // the N tile, K of the K tile, M at least one M tile.
  void* bt = nullptr;
  int64_t ldbt = 0;
};

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s);

// bf16 dst[c * ld_dst + r] = src[r * ld_src + c] for r < rows, c < cols.
hipError_t launch_transpose_bf16(const void* src, int64_t rows, int64_t cols, int64_t ld_src,
                                 void* dst, int64_t ld_dst, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s);

}  // namespace fljsd
