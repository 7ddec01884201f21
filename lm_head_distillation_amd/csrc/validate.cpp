// Argument checks and the pure host entry points (see validate.h). Every
// check runs before the first HIP call of an entry point, so an error leaves
// every output untouched.
#include "validate.h"

#include <cmath>
#include <cstdint>
#include <string>

namespace fljsd {
namespace {

thread_local std::string g_last_error;

bool known_dtype(int dtype) { return dtype == FLJSD_F32 || dtype == FLJSD_BF16; }
bool known_reduction(int r) { return r >= FLJSD_BATCHMEAN && r <= FLJSD_NONE; }

// Sizes the planner accepts: positive and at most kMaxPlanDim, so no
// intermediate of the plan arithmetic overflows (the workspace total itself
// saturates, see plan.cpp).
bool plannable(int64_t x) { return x > 0 && x <= kMaxPlanDim; }

int check_common(int dtype, float beta, float temperature, int reduction) {
  if (!known_dtype(dtype)) return fail(FLJSD_EDTYPE, "unknown dtype");
  if (!known_reduction(reduction)) return fail(FLJSD_EDTYPE, "unknown reduction");
  if (!(beta >= 0.0f && beta <= 1.0f)) return fail(FLJSD_EINVAL, "beta must be in [0, 1]");
  if (!(temperature > 0.0f) || !std::isfinite(temperature))
    return fail(FLJSD_EINVAL, "temperature must be finite and > 0");
  return FLJSD_OK;
}

int check_aligned(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(FLJSD_EALIGN, "pointers must be 16-byte aligned");
  return FLJSD_OK;
}

int check_workspace_total(const void* workspace, size_t workspace_bytes, size_t total) {
  if (total == kSizeOverflow) return fail(FLJSD_EWORKSPACE, "the workspace size overflows size_t");
  if (!workspace) return fail(FLJSD_EINVAL, "workspace must not be NULL");
  if (workspace_bytes < total)
    return fail(FLJSD_EWORKSPACE, "workspace needs " + std::to_string(total) + " bytes");
  return FLJSD_OK;
}

}  // namespace

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

void clear_last_error() { g_last_error.clear(); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_forward_backward(const void* X_s, const void* W_s, const void* X_t, const void* W_t,
                           int64_t BT, int64_t H_s, int64_t H_t, int64_t V, int dtype, float beta,
                           float temperature, int reduction, int num_chunks, const float* loss,
                           const void* grad_X_s, const void* grad_W_s, int grad_w_dtype,
                           unsigned flags, const void* workspace, size_t workspace_bytes,
                           ChunkPlan* plan) {
  if (!X_s || !W_s || !X_t || !W_t || !loss)
    return fail(FLJSD_EINVAL, "X_s, W_s, X_t, W_t and loss must not be NULL");
  if (BT <= 0 || H_s <= 0 || H_t <= 0 || V <= 0)
    return fail(FLJSD_EINVAL, "BT, H_s, H_t and V must be > 0");
  if (BT > INT32_MAX || V > INT32_MAX) return fail(FLJSD_EINVAL, "BT and V must fit in int32");
  if (H_s > kMaxPlanDim || H_t > kMaxPlanDim) return fail(FLJSD_EINVAL, "H_s or H_t too large");
  int rc = check_common(dtype, beta, temperature, reduction);
  if (rc != FLJSD_OK) return rc;
  if (num_chunks < 0) return fail(FLJSD_EINVAL, "num_chunks must be >= 0");
  if (grad_w_dtype != dtype && !(dtype == FLJSD_BF16 && grad_w_dtype == FLJSD_F32))
    return fail(FLJSD_EDTYPE, "grad_w_dtype must equal dtype, or be F32 with BF16 inputs");
  if (flags & ~static_cast<unsigned>(FLJSD_ACCUMULATE_GRAD_W | FLJSD_TEMPERATURE_SQUARED))
    return fail(FLJSD_EINVAL, "unknown flag bits");
  rc = check_aligned({X_s, W_s, X_t, W_t, loss, grad_X_s, grad_W_s, workspace});
  if (rc != FLJSD_OK) return rc;
  const int vec = dtype_vec(dtype);
  if (H_s % vec != 0 || H_t % vec != 0)
    return fail(FLJSD_EALIGN, "H_s and H_t must be multiples of 16 bytes of elements");
  int64_t nc = num_chunks;
  if (nc == 0) {
    nc = policy_num_chunks(BT, H_s, H_t, V, dtype, workspace_bytes);
    if (nc <= 0) return fail(FLJSD_EWORKSPACE, "no chunk count fits the workspace");
  }
  *plan = plan_chunks(BT, H_s, H_t, V, dtype, nc);
  // W_s^T only serves grad_input, and only when the workspace has room for it.
  if (plan->w_transposed && (!grad_X_s || workspace_bytes < plan->total)) drop_w_transposed(plan);
  return check_workspace_total(workspace, workspace_bytes, plan->total);
}

int check_generalized_jsd_args(const void* logits_s, const void* logits_t, int64_t BT, int64_t V,
                               int64_t ld, int dtype, float beta, float temperature,
                               int reduction, const float* loss, const void* grad_logits_s) {
  if (!logits_s || !logits_t || !loss)
    return fail(FLJSD_EINVAL, "logits_s, logits_t and loss must not be NULL");
  if (BT <= 0 || V <= 0) return fail(FLJSD_EINVAL, "BT and V must be > 0");
  if (BT > INT32_MAX || V > INT32_MAX) return fail(FLJSD_EINVAL, "BT and V must fit in int32");
  if (ld < V) return fail(FLJSD_EINVAL, "ld must be >= V");
  int rc = check_common(dtype, beta, temperature, reduction);
  if (rc != FLJSD_OK) return rc;
  return check_aligned({logits_s, logits_t, loss, grad_logits_s});
}

int check_jsd_workspace(int64_t BT, int64_t V, const void* workspace, size_t workspace_bytes,
                        JsdPlan* plan) {
  if (workspace && !aligned16(workspace))
    return fail(FLJSD_EALIGN, "pointers must be 16-byte aligned");
  *plan = plan_jsd(BT, V);
  return check_workspace_total(workspace, workspace_bytes, plan->total);
}

int check_noalloc_scratch(int64_t BT, int64_t V, size_t scratch_bytes) {
  const size_t need = plan_jsd(BT, V).total;
  if (need > scratch_bytes)
    return fail(FLJSD_EWORKSPACE, "this shape needs " + std::to_string(need) +
                                      " bytes of scratch; the no-allocation entry point holds " +
                                      std::to_string(scratch_bytes));
  return FLJSD_OK;
}

int check_elem_loss(const void* a, const void* b, int64_t BT, int64_t V, int64_t ld, int dtype,
                    int reduction, bool check_beta, float beta, const float* loss,
                    const void* grad, const void* workspace, size_t workspace_bytes,
                    JsdPlan* plan) {
  if (check_beta && !(beta >= 0.0f && beta <= 1.0f))
    return fail(FLJSD_EINVAL, "beta must be in [0, 1]");
  if (!a || !b || !loss) return fail(FLJSD_EINVAL, "inputs and loss must not be NULL");
  if (BT <= 0 || V <= 0) return fail(FLJSD_EINVAL, "BT and V must be > 0");
  if (BT > INT32_MAX || V > INT32_MAX) return fail(FLJSD_EINVAL, "BT and V must fit in int32");
  if (ld < V) return fail(FLJSD_EINVAL, "ld must be >= V");
  if (!known_dtype(dtype)) return fail(FLJSD_EDTYPE, "unknown dtype");
  if (!known_reduction(reduction)) return fail(FLJSD_EDTYPE, "unknown reduction");
  const int rc = check_aligned({a, b, loss, grad, workspace});
  if (rc != FLJSD_OK) return rc;
  *plan = plan_jsd(BT, V);
  return check_workspace_total(workspace, workspace_bytes, plan->total);
}

int check_flce(const void* X, const void* W, const int64_t* labels, int64_t BT, int64_t H,
               int64_t V, int dtype, float label_smoothing, int reduction, int num_chunks,
               const float* loss, const void* grad_X, const void* grad_W, int grad_w_dtype,
               unsigned flags, const void* workspace, size_t workspace_bytes, CePlan* plan) {
  if (!X || !W || !labels || !loss) return fail(FLJSD_EINVAL, "X, W, labels and loss must not be NULL");
  if (BT <= 0 || H <= 0 || V <= 0) return fail(FLJSD_EINVAL, "BT, H and V must be > 0");
  if (BT > INT32_MAX || V > INT32_MAX) return fail(FLJSD_EINVAL, "BT and V must fit in int32");
  if (H > kMaxPlanDim) return fail(FLJSD_EINVAL, "H too large");
  if (!known_dtype(dtype)) return fail(FLJSD_EDTYPE, "unknown dtype");
  if (!known_reduction(reduction)) return fail(FLJSD_EDTYPE, "unknown reduction");
  if (!(label_smoothing >= 0.0f && label_smoothing <= 1.0f))
    return fail(FLJSD_EINVAL, "label_smoothing must be in [0, 1]");
  if (num_chunks < 0) return fail(FLJSD_EINVAL, "num_chunks must be >= 0");
  if (grad_w_dtype != dtype && !(dtype == FLJSD_BF16 && grad_w_dtype == FLJSD_F32))
    return fail(FLJSD_EDTYPE, "grad_w_dtype must equal dtype, or be F32 with BF16 inputs");
  if (flags & ~static_cast<unsigned>(FLJSD_ACCUMULATE_GRAD_W))
    return fail(FLJSD_EINVAL, "unknown flag bits");
  int rc = check_aligned({X, W, loss, grad_X, grad_W, workspace});
  if (rc != FLJSD_OK) return rc;
  if ((reinterpret_cast<uintptr_t>(labels) & 7u) != 0)
    return fail(FLJSD_EALIGN, "labels must be 8-byte aligned");
  if (H % dtype_vec(dtype) != 0) return fail(FLJSD_EALIGN, "H must be a multiple of 16 bytes of elements");
  int64_t nc = num_chunks;
  if (nc == 0) {
    nc = policy_num_chunks_ce(BT, H, V, dtype, workspace_bytes);
    if (nc <= 0) return fail(FLJSD_EWORKSPACE, "no chunk count fits the workspace");
  }
  *plan = plan_ce_chunks(BT, H, V, dtype, nc);
  if (plan->w_transposed && (!grad_X || workspace_bytes < plan->total)) drop_w_transposed(plan);
  return check_workspace_total(workspace, workspace_bytes, plan->total);
}

}  // namespace fljsd

using namespace fljsd;

// A total that overflows size_t is reported as 0, like any other shape the
// library cannot run.
FLJSD_EXPORT size_t fljsd_workspace_size(int64_t BT, int64_t H_s, int64_t H_t, int64_t V,
                                         int dtype, int num_chunks) {
  if (!plannable(BT) || !plannable(H_s) || !plannable(H_t) || !plannable(V) || num_chunks < 1)
    return 0;
  if (!known_dtype(dtype)) return 0;
  const size_t total = plan_chunks(BT, H_s, H_t, V, dtype, num_chunks).total;
  return total == kSizeOverflow ? 0 : total;
}

FLJSD_EXPORT size_t fljsd_generalized_jsd_workspace_size(int64_t BT, int64_t V, int dtype) {
  if (!plannable(BT) || !plannable(V)) return 0;
  if (!known_dtype(dtype)) return 0;
  const size_t total = plan_jsd(BT, V).total;
  return total == kSizeOverflow ? 0 : total;
}

FLJSD_EXPORT int fljsd_plan_num_chunks(int64_t BT, int64_t H_s, int64_t H_t, int64_t V,
                                       int dtype, size_t budget_bytes) {
  clear_last_error();
  if (BT <= 0 || H_s <= 0 || H_t <= 0 || V <= 0) return fail(FLJSD_EINVAL, "sizes must be > 0");
  if (!plannable(BT) || !plannable(H_s) || !plannable(H_t) || !plannable(V))
    return fail(FLJSD_EINVAL, "sizes too large to plan");
  if (!known_dtype(dtype)) return fail(FLJSD_EDTYPE, "unknown dtype");
  const int64_t nc = policy_num_chunks(BT, H_s, H_t, V, dtype, budget_bytes);
  if (nc <= 0) return fail(FLJSD_EWORKSPACE, "no chunk count fits the budget");
  if (nc > INT32_MAX) return fail(FLJSD_EINVAL, "chunk count overflows int");
  return static_cast<int>(nc);
}

FLJSD_EXPORT size_t fljsd_flce_workspace_size(int64_t BT, int64_t H, int64_t V, int dtype,
                                              int num_chunks) {
  if (!plannable(BT) || !plannable(H) || !plannable(V) || num_chunks < 1) return 0;
  if (!known_dtype(dtype)) return 0;
  const size_t total = plan_ce_chunks(BT, H, V, dtype, num_chunks).total;
  return total == kSizeOverflow ? 0 : total;
}

FLJSD_EXPORT int fljsd_flce_plan_num_chunks(int64_t BT, int64_t H, int64_t V, int dtype,
                                            size_t budget_bytes) {
  clear_last_error();
  if (BT <= 0 || H <= 0 || V <= 0) return fail(FLJSD_EINVAL, "sizes must be > 0");
  if (!plannable(BT) || !plannable(H) || !plannable(V))
    return fail(FLJSD_EINVAL, "sizes too large to plan");
  if (!known_dtype(dtype)) return fail(FLJSD_EDTYPE, "unknown dtype");
  const int64_t nc = policy_num_chunks_ce(BT, H, V, dtype, budget_bytes);
  if (nc <= 0) return fail(FLJSD_EWORKSPACE, "no chunk count fits the budget");
  if (nc > INT32_MAX) return fail(FLJSD_EINVAL, "chunk count overflows int");
  return static_cast<int>(nc);
}

FLJSD_EXPORT const char* fljsd_strerror(int code) {
  switch (code) {
    case FLJSD_OK: return "success";
    case FLJSD_EINVAL: return "invalid argument";
    case FLJSD_EDTYPE: return "unsupported dtype or reduction";
    case FLJSD_EWORKSPACE: return "workspace too small";
    case FLJSD_EALIGN: return "misaligned pointer or leading dimension";
    case FLJSD_EHIP: return "HIP runtime error";
    case FLJSD_EDEVICE: return "device is not an MI355X (gfx950)";
    default: return "unknown status code";
  }
}

FLJSD_EXPORT const char* fljsd_last_error(void) { return g_last_error.c_str(); }
