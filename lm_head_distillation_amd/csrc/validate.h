// Argument checks of the C-ABI entry points, and the pure host functions the
// header exports (workspace sizes, chunk policies, status strings). No HIP
// here: this code builds with a host compiler alone, which is how the test
// suite also runs it under AddressSanitizer and UndefinedBehaviorSanitizer.
// Each check returns FLJSD_OK or a negative status code, and on failure
// records a message for fljsd_last_error().
#pragma once

#include "fljsd.h"
#include "plan.h"

#include <cstddef>
#include <cstdint>
#include <string>

#ifndef FLJSD_EXPORT
#define FLJSD_EXPORT extern "C" __attribute__((visibility("default")))
#endif

namespace fljsd {

// Records `msg` as the calling thread's last error and returns `code`.
int fail(int code, const std::string& msg);
void clear_last_error();
bool aligned16(const void* p);

// fljsd_forward_backward_ex: every argument, then the chunk plan (num_chunks
// 0 picks the policy's count for workspace_bytes) and the workspace size.
int check_forward_backward(const void* X_s, const void* W_s, const void* X_t, const void* W_t,
                           int64_t BT, int64_t H_s, int64_t H_t, int64_t V, int dtype, float beta,
                           float temperature, int reduction, int num_chunks, const float* loss,
                           const void* grad_X_s, const void* grad_W_s, int grad_w_dtype,
                           unsigned flags, const void* workspace, size_t workspace_bytes,
                           ChunkPlan* plan);

// fljsd_generalized_jsd(_noalloc): every argument except the workspace.
int check_generalized_jsd_args(const void* logits_s, const void* logits_t, int64_t BT, int64_t V,
                               int64_t ld, int dtype, float beta, float temperature,
                               int reduction, const float* loss, const void* grad_logits_s);

// The loss passes' workspace (caller's or the library's scratch array).
int check_jsd_workspace(int64_t BT, int64_t V, const void* workspace, size_t workspace_bytes,
                        JsdPlan* plan);

// fljsd_generalized_jsd_noalloc: the shape's workspace within the scratch array.
int check_noalloc_scratch(int64_t BT, int64_t V, size_t scratch_bytes);

// fljsd_jsd_logprob (check_beta) and fljsd_tvd.
int check_elem_loss(const void* a, const void* b, int64_t BT, int64_t V, int64_t ld, int dtype,
                    int reduction, bool check_beta, float beta, const float* loss,
                    const void* grad, const void* workspace, size_t workspace_bytes,
                    JsdPlan* plan);

// fljsd_flce_forward_backward.
int check_flce(const void* X, const void* W, const int64_t* labels, int64_t BT, int64_t H,
               int64_t V, int dtype, float label_smoothing, int reduction, int num_chunks,
               const float* loss, const void* grad_X, const void* grad_W, int grad_w_dtype,
               unsigned flags, const void* workspace, size_t workspace_bytes, CePlan* plan);

}  // namespace fljsd
