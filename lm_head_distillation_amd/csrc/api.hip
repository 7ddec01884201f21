// C-ABI entry points: argument checks, planning, and the stream-ordered launch
// sequence of the fused-linear JSD pass. See include/fljsd.h for the contract.
//
// Per chunk of C rows (Liger-Kernel PR #1352, Details; PR #1429, Summary):
//   Z_s = X_s W_s^T, Z_t = X_t W_t^T             two logits GEMMs
//   pass 1 / pass 2 / pass 3                      online-softmax JSD, dZ over Z_s
//   grad_X_s[chunk] = dZ W_s                      (split-K when few output tiles)
//   grad_W_s = dZ^T X_s[chunk]                    overwrite on chunk 0, else add
// then one scalar reduction of the per-row losses.
#include "fljsd.h"
#include "kernels.h"
#include "plan.h"
#include "validate.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>


namespace fljsd {
namespace {

int fail_hip(hipError_t e, const char* what) {
  return fail(FLJSD_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

double reduction_scale(int reduction, int64_t rows, int64_t V) {
  switch (reduction) {
    case FLJSD_BATCHMEAN: return 1.0 / static_cast<double>(rows);
    case FLJSD_MEAN: return 1.0 / (static_cast<double>(rows) * static_cast<double>(V));
    default: return 1.0;  // SUM, NONE
  }
}

int mode_for(float beta) {
  if (beta == 0.0f) return kModeForwardKL;
  if (beta == 1.0f) return kModeReverseKL;
  return kModeGeneralized;
}

// ---- device check (once per device) ---------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FLJSD_EDEVICE, "device index out of range");
  int state = g_device_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDeviceProperties");
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_ok[dev].store(state, std::memory_order_release);
    if (state == 2) return fail(FLJSD_EDEVICE, std::string("device is ") + prop.gcnArchName);
  }
  return state == 1 ? FLJSD_OK : fail(FLJSD_EDEVICE, "device is not gfx950");
}

// ---- kernel timing ----------------------------------------------------------
struct ProfRecord {
  hipEvent_t start, stop;
  int cls;
  double flops, bytes;
};

struct Profiler {
  bool enabled = false;
  std::vector<hipEvent_t> pool;
  size_t next = 0;
  std::vector<ProfRecord> records;
  double ms[FLJSD_KCLASS_COUNT] = {};
  double flops[FLJSD_KCLASS_COUNT] = {};
  double bytes[FLJSD_KCLASS_COUNT] = {};
  int64_t launches[FLJSD_KCLASS_COUNT] = {};

  void clear() {
    records.clear();
    next = 0;
    for (int i = 0; i < FLJSD_KCLASS_COUNT; ++i) {
      ms[i] = flops[i] = bytes[i] = 0.0;
      launches[i] = 0;
    }
  }
  hipError_t take(hipEvent_t* ev) {
    if (next == pool.size()) {
      hipEvent_t e;
      hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) return err;
      pool.push_back(e);
    }
    *ev = pool[next++];
    return hipSuccess;
  }
};

Profiler g_prof;

// Launch `f` on `s`, bracketed by timing events when profiling is on.
template <class F>
hipError_t timed(hipStream_t s, int cls, double flops, double bytes, F&& f) {
  if (!g_prof.enabled) return f();
  ProfRecord rec{};
  rec.cls = cls;
  rec.flops = flops;
  rec.bytes = bytes;
  hipError_t e = g_prof.take(&rec.start);
  if (e == hipSuccess) e = g_prof.take(&rec.stop);
  if (e == hipSuccess) e = hipEventRecord(rec.start, s);
  if (e != hipSuccess) return e;
  e = f();
  if (e != hipSuccess) return e;
  e = hipEventRecord(rec.stop, s);
  if (e == hipSuccess) g_prof.records.push_back(rec);
  return e;
}

hipError_t gemm(int dtype, const GemmArgs& g, hipStream_t s) {
  return dtype == FLJSD_BF16 ? launch_gemm_bf16(g, s) : launch_gemm_f32(g, s);
}

double gemm_bytes(const GemmArgs& g, int es) {
  const double in = (static_cast<double>(g.M) * g.K + static_cast<double>(g.N) * g.K) * es;
  const bool f32_out = g.epilogue == kEpiPartialF32 || g.epilogue == kEpiAccumulateF32;
  const bool rmw = g.epilogue == kEpiAccumulate || g.epilogue == kEpiAccumulateF32;
  const double out = static_cast<double>(g.M) * g.N * (f32_out ? 4.0 : es) * (rmw ? 2 : 1);
  return in + out;
}

// The three loss passes. With `part_s` the row statistics come from the
// logits GEMMs' partials (a merge over `tiles` per row) instead of pass 1's
// read of both rows.
int run_jsd_passes(const JsdArgs& ja, int dtype, bool write_grad, int64_t V, int es,
                   hipStream_t s, const float2* part_s = nullptr, const float2* part_t = nullptr,
                   int64_t tiles = 0, void* dzt = nullptr, int64_t ldt = 0) {
  const double row_bytes = static_cast<double>(ja.rows) * V * es;
  hipError_t e;
  if (part_s) {
    e = timed(s, FLJSD_KCLASS_JSD_STATS, 0.0, 16.0 * ja.rows * tiles,
              [&] { return launch_jsd_stats_merge(ja, part_s, part_t, tiles, s); });
  } else {
    e = timed(s, FLJSD_KCLASS_JSD_STATS, 0.0, 2 * row_bytes,
              [&] { return launch_jsd_stats(ja, dtype, s); });
  }
  if (e != hipSuccess) return fail_hip(e, "launch jsd_stats");
  // bf16 with the transposed gradient: pass 3 also sums the loss terms (not
  // the reverse KL, whose row loss is its G), so pass 2 computes only G, and
  // the forward KL, which needs no G, has no pass 2.
  const bool loss_in_pass3 = write_grad && dzt && ja.mode != kModeReverseKL;
  if (!(loss_in_pass3 && ja.mode == kModeForwardKL)) {
    e = timed(s, FLJSD_KCLASS_JSD_LOSS, 0.0, 2 * row_bytes, [&] {
      return loss_in_pass3 ? launch_jsd_gsum(ja, s) : launch_jsd_loss(ja, dtype, s);
    });
    if (e != hipSuccess) return fail_hip(e, "launch jsd_loss");
  }
  if (write_grad && dzt) {
    e = timed(s, FLJSD_KCLASS_JSD_GRAD, 0.0, 4 * row_bytes,
              [&] { return launch_jsd_grad_transposed(ja, dzt, ldt, loss_in_pass3, s); });
    if (e != hipSuccess) return fail_hip(e, "launch jsd_grad");
    if (loss_in_pass3) {
      int64_t span = 0, nblk = 0;
      grad_t_geometry(ja.rows, V, &span, &nblk);
      e = timed(s, FLJSD_KCLASS_LOSS_REDUCE, 0.0, 4.0 * ja.rows * (nblk + 1),
                [&] { return launch_jsd_row_loss_merge(ja, s); });
      if (e != hipSuccess) return fail_hip(e, "launch row loss merge");
    }
  } else if (write_grad) {
    e = timed(s, FLJSD_KCLASS_JSD_GRAD, 0.0, 3 * row_bytes,
              [&] { return launch_jsd_grad(ja, dtype, s); });
    if (e != hipSuccess) return fail_hip(e, "launch jsd_grad");
  } else {
    e = launch_jsd_row_loss(ja, s);
    if (e != hipSuccess) return fail_hip(e, "launch jsd_row_loss");
  }
  return FLJSD_OK;
}

// ---- the per-chunk GEMMs shared by the JSD and cross-entropy passes --------

// Z[rows, ldz] = X[rows, H] W[V, H]^T, rounded once to the dtype. With
// `stat_part` (bf16), also each row's statistics per N-tile of the rounded
// logits (max, sum 2^((z - max) stat_k)) into stat_part [rows, stat_tiles].
// With `wt` (bf16, shapes that tile evenly), the product also writes
// W^T [H, ldwt] from the W tiles its first M-tile's workgroups hold in LDS.
int run_logits_gemm(int dtype, const void* X, const void* W, void* Z, int64_t rows, int64_t V,
                    int64_t H, int64_t ldz, hipStream_t s, float2* stat_part = nullptr,
                    int64_t stat_tiles = 0, float stat_k = 0.f, void* wt = nullptr,
                    int64_t ldwt = 0) {
  GemmArgs g;
  g.A = X;
  g.B = W;
  g.C = Z;
  g.M = rows;
  g.N = V;
  g.K = H;
  g.lda = H;
  g.ldb = H;
  g.ldc = ldz;
  g.a_kcontig = true;
  g.b_kcontig = true;
  g.epilogue = stat_part ? kEpiStoreStats : kEpiStore;
  g.stat_part = stat_part;
  g.stat_ld = stat_tiles;
  g.stat_k = stat_k;
  g.splitk = 1;
  g.k_per_split = H;
  g.group_m = 4;
  g.bt = wt;
  g.ldbt = ldwt;
  const double side_bytes = wt ? static_cast<double>(V) * H * dtype_size(dtype) : 0.0;
  hipError_t e = timed(s, FLJSD_KCLASS_GEMM_LOGITS, 2.0 * rows * V * H,
                       gemm_bytes(g, dtype_size(dtype)) + side_bytes,
                       [&] { return gemm(dtype, g, s); });
  return e == hipSuccess ? FLJSD_OK : fail_hip(e, "launch logits GEMM");
}

// gx[rows, H] = dZ[rows, ldz] W[V, H]; bf16 splits K when the output has few
// tiles, summing fp32 partials (in `partial`) in split order. With `wt`
// (W^T [H, ldwt]) both operands are K-contiguous.
int run_grad_input(int dtype, const void* dZ, int64_t ldz, const void* W, int64_t rows,
                   int64_t H, int64_t V, void* gx, int splitk, int64_t k_per_split,
                   void* partial, hipStream_t s, const void* wt = nullptr, int64_t ldwt = 0) {
  const int es = dtype_size(dtype);
  GemmArgs g;
  g.A = dZ;
  g.B = wt ? wt : W;
  g.M = rows;
  g.N = H;
  g.K = V;
  g.lda = ldz;
  g.ldb = wt ? ldwt : H;
  g.ldc = H;
  g.a_kcontig = true;
  g.b_kcontig = wt != nullptr;
  g.group_m = 8;
  const bool split = dtype == FLJSD_BF16 && splitk > 1;
  if (split) {
    g.C = partial;
    g.epilogue = kEpiPartialF32;
    g.splitk = splitk;
    g.k_per_split = k_per_split;
  } else {
    g.C = gx;
    g.epilogue = kEpiStore;
    g.splitk = 1;
    g.k_per_split = V;
  }
  hipError_t e = timed(s, FLJSD_KCLASS_GEMM_GRAD_INPUT, 2.0 * rows * H * V, gemm_bytes(g, es),
                       [&] { return gemm(dtype, g, s); });
  if (e != hipSuccess) return fail_hip(e, "launch grad_input GEMM");
  if (split) {
    const double red_bytes = static_cast<double>(rows) * H * (4.0 * splitk + es);
    e = timed(s, FLJSD_KCLASS_SPLITK_REDUCE, 0.0, red_bytes, [&] {
      return launch_splitk_reduce(static_cast<const float*>(partial), splitk, rows, H, gx, H,
                                  dtype, s);
    });
    if (e != hipSuccess) return fail_hip(e, "launch split-K reduce");
  }
  return FLJSD_OK;
}

// gW[V, H] (epilogue: store or add, bf16 or fp32) = dZ[rows, ldz]^T X[rows, H].
// `transposed`: first write dZ^T [V, ldt] to dzt and X^T [H, ldt] to xt, so
// both operands are K-contiguous for the direct-copy matrix-core path.
int run_grad_weight(int dtype, const void* dZ, int64_t ldz, const void* X, int64_t rows,
                    int64_t H, int64_t V, void* gW, bool transposed, void* dzt, void* xt,
                    int64_t ldt, int epilogue, hipStream_t s, bool dz_transposed = false) {
  const int es = dtype_size(dtype);
  GemmArgs g;
  if (transposed) {
    const double tbytes = 2.0 * static_cast<double>(rows) * ((dz_transposed ? 0 : V) + H) * es;
    hipError_t e = timed(s, FLJSD_KCLASS_TRANSPOSE, 0.0, tbytes, [&] {
      if (!dz_transposed) {
        hipError_t t = launch_transpose_bf16(dZ, rows, V, ldz, dzt, ldt, s);
        if (t != hipSuccess) return t;
      }
      return launch_transpose_bf16(X, rows, H, H, xt, ldt, s);
    });
    if (e != hipSuccess) return fail_hip(e, "launch transpose");
    g.A = dzt;                    // A(m=v, k=r) = dZ^T[v, r]
    g.B = xt;                     // B(n=h, k=r) = X^T[h, r]
    g.lda = ldt;
    g.ldb = ldt;
    g.a_kcontig = true;
    g.b_kcontig = true;
  } else {
    g.A = dZ;                     // A(m=v, k=r) = dZ[r, v]
    g.B = X;                      // B(n=h, k=r) = X[r, h]
    g.lda = ldz;
    g.ldb = H;
    g.a_kcontig = false;
    g.b_kcontig = false;
  }
  g.C = gW;
  g.M = V;
  g.N = H;
  g.K = rows;
  g.ldc = H;
  g.epilogue = epilogue;
  g.splitk = 1;
  g.k_per_split = rows;
  g.group_m = 4;   // an XCD's concurrent 256 x 256 tiles: 4 M x 8 N (measured best of 1..16)
  g.wgrad = true;
  hipError_t e = timed(s, FLJSD_KCLASS_GEMM_GRAD_WEIGHT, 2.0 * rows * H * V, gemm_bytes(g, es),
                       [&] { return gemm(dtype, g, s); });
  return e == hipSuccess ? FLJSD_OK : fail_hip(e, "launch grad_weight GEMM");
}

}  // namespace
}  // namespace fljsd

using namespace fljsd;

FLJSD_EXPORT int fljsd_profile_enable(int enable) {
  g_prof.enabled = enable != 0;
  g_prof.clear();
  return FLJSD_OK;
}

FLJSD_EXPORT int fljsd_profile_read(double* total_ms, int64_t* launches, double* flops,
                                    double* hbm_bytes, int n) {
  for (const ProfRecord& r : g_prof.records) {
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return fail_hip(e, "hipEventElapsedTime");
    g_prof.ms[r.cls] += ms;
    g_prof.flops[r.cls] += r.flops;
    g_prof.bytes[r.cls] += r.bytes;
    g_prof.launches[r.cls] += 1;
  }
  g_prof.records.clear();
  g_prof.next = 0;
  for (int i = 0; i < n && i < FLJSD_KCLASS_COUNT; ++i) {
    if (total_ms) total_ms[i] = g_prof.ms[i];
    if (launches) launches[i] = g_prof.launches[i];
    if (flops) flops[i] = g_prof.flops[i];
    if (hbm_bytes) hbm_bytes[i] = g_prof.bytes[i];
  }
  return FLJSD_OK;
}

FLJSD_EXPORT int fljsd_forward_backward(const void* X_s, const void* W_s, const void* X_t,
                                        const void* W_t, int64_t BT, int64_t H_s, int64_t H_t,
                                        int64_t V, int dtype, float beta, float temperature,
                                        int reduction, int num_chunks, float* loss,
                                        void* grad_X_s, void* grad_W_s, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return fljsd_forward_backward_ex(X_s, W_s, X_t, W_t, BT, H_s, H_t, V, dtype, beta, temperature,
                                   reduction, num_chunks, loss, grad_X_s, grad_W_s, dtype, 0u,
                                   workspace, workspace_bytes, stream);
}

FLJSD_EXPORT int fljsd_forward_backward_ex(const void* X_s, const void* W_s, const void* X_t,
                                           const void* W_t, int64_t BT, int64_t H_s,
                                           int64_t H_t, int64_t V, int dtype, float beta,
                                           float temperature, int reduction, int num_chunks,
                                           float* loss, void* grad_X_s, void* grad_W_s,
                                           int grad_w_dtype, unsigned flags, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  clear_last_error();
  ChunkPlan plan;
  int rc = check_forward_backward(X_s, W_s, X_t, W_t, BT, H_s, H_t, V, dtype, beta, temperature,
                                  reduction, num_chunks, loss, grad_X_s, grad_W_s, grad_w_dtype,
                                  flags, workspace, workspace_bytes, &plan);
  if (rc != FLJSD_OK) return rc;
  const bool gw_f32_acc = dtype == FLJSD_BF16 && grad_w_dtype == FLJSD_F32;
  const bool gw_add_existing = (flags & FLJSD_ACCUMULATE_GRAD_W) != 0;
  rc = check_device();
  if (rc != FLJSD_OK) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int es = dtype_size(dtype);
  char* ws = static_cast<char*>(workspace);
  void* Zs = ws + plan.off_zs;
  void* Zt = ws + plan.off_zt;
  float* row_loss = reduction == FLJSD_NONE ? loss : reinterpret_cast<float*>(ws + plan.off_row_loss);
  const double scale = reduction_scale(reduction, BT, V);
  const bool write_grad = grad_X_s != nullptr || grad_W_s != nullptr;

  JsdArgs ja;
  ja.zs = Zs;
  ja.zt = Zt;
  ja.grad = Zs;  // dZ replaces the student logits in place
  ja.ld = plan.ldz;
  ja.vec_ok = true;  // ldz is a multiple of 8 elements
  ja.V = V;
  ja.slice_w = plan.slices.slice_w;
  ja.S = plan.slices.S;
  ja.k2 = static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
  ja.beta = beta;
  // The optional T^2 factor (PR #1352, Open question 2) multiplies the loss
  // and, with it, every gradient.
  const double t2 = (flags & FLJSD_TEMPERATURE_SQUARED)
                        ? static_cast<double>(temperature) * static_cast<double>(temperature)
                        : 1.0;
  ja.grad_scale = static_cast<float>(scale * t2 / static_cast<double>(temperature));
  ja.row_scale = static_cast<float>(t2);
  ja.mode = mode_for(beta);
  ja.stats = reinterpret_cast<float4*>(ws + plan.off_stats);
  ja.lg = reinterpret_cast<float2*>(ws + plan.off_lg);
  ja.peak = reinterpret_cast<float4*>(ws + plan.off_peak);
  ja.ref = reinterpret_cast<float*>(ws + plan.off_ref);
  ja.lpart = reinterpret_cast<float*>(ws + plan.off_lpart);

  const char* Xs = static_cast<const char*>(X_s);
  const char* Xt = static_cast<const char*>(X_t);
  for (int64_t ci = 0; ci < plan.n_chunks; ++ci) {
    const int64_t r0 = ci * plan.C;
    const int64_t rows = std::min(plan.C, BT - r0);

    float2* part_s = plan.gemm_stats ? reinterpret_cast<float2*>(ws + plan.off_spart) : nullptr;
    float2* part_t = plan.gemm_stats ? part_s + plan.C * plan.stat_tiles : nullptr;
    // W_s^T for grad_input, written once, by the first chunk's product.
    void* wst = (grad_X_s && plan.w_transposed) ? ws + plan.off_wst : nullptr;
    rc = run_logits_gemm(dtype, Xs + r0 * H_s * es, W_s, Zs, rows, V, H_s, plan.ldz, s, part_s,
                         plan.stat_tiles, ja.k2, ci == 0 ? wst : nullptr, plan.ldz);
    if (rc == FLJSD_OK)
      rc = run_logits_gemm(dtype, Xt + r0 * H_t * es, W_t, Zt, rows, V, H_t, plan.ldz, s, part_t,
                           plan.stat_tiles, ja.k2);
    if (rc != FLJSD_OK) return rc;

    ja.rows = rows;
    ja.row_loss = row_loss + r0;
    // With a weight gradient on the transposed path, pass 3 also writes dZ^T.
    void* dzt = (grad_W_s && plan.transposed_grad_w) ? ws + plan.off_dzt : nullptr;
    rc = run_jsd_passes(ja, dtype, write_grad, V, es, s, part_s, part_t, plan.stat_tiles, dzt,
                        plan.ldt);
    if (rc != FLJSD_OK) return rc;

    if (grad_X_s) {
      rc = run_grad_input(dtype, Zs, plan.ldz, W_s, rows, H_s, V,
                          static_cast<char*>(grad_X_s) + r0 * H_s * es, plan.splitk,
                          plan.k_per_split, ws + plan.off_partial, s, wst, plan.ldz);
      if (rc != FLJSD_OK) return rc;
    }

    if (grad_W_s) {
      // Chunk 0 overwrites unless the caller asked to add to grad_W's
      // contents; later chunks add. An fp32 grad_W takes the bf16 product
      // unrounded (one-split fp32 store, or fp32 read-add-write). With bf16
      // inputs pass 3 has already written dZ^T (its own workspace region).
      const bool add = ci > 0 || gw_add_existing;
      const int epi = gw_f32_acc ? (add ? kEpiAccumulateF32 : kEpiPartialF32)
                                 : (add ? kEpiAccumulate : kEpiStore);
      rc = run_grad_weight(dtype, Zs, plan.ldz, Xs + r0 * H_s * es, rows, H_s, V, grad_W_s,
                           plan.transposed_grad_w, ws + plan.off_dzt, ws + plan.off_xt, plan.ldt,
                           epi, s, /*dz_transposed=*/true);
      if (rc != FLJSD_OK) return rc;
    }
  }

  if (reduction != FLJSD_NONE) {
    hipError_t e = timed(s, FLJSD_KCLASS_LOSS_REDUCE, 0.0, 4.0 * BT,
                         [&] { return launch_loss_reduce(row_loss, BT, static_cast<float>(scale), loss, s); });
    if (e != hipSuccess) return fail_hip(e, "launch loss reduce");
  }
  return FLJSD_OK;
}

namespace fljsd {
namespace {

// fljsd_generalized_jsd with the workspace already chosen (the caller's, or
// the no-allocation entry point's file-scope scratch array).
int generalized_jsd_impl(const void* logits_s, const void* logits_t, int64_t BT, int64_t V,
                         int64_t ld, int dtype, float beta, float temperature, int reduction,
                         float* loss, void* grad_logits_s, void* workspace,
                         size_t workspace_bytes, void* stream) {
  int rc = check_generalized_jsd_args(logits_s, logits_t, BT, V, ld, dtype, beta, temperature,
                                      reduction, loss, grad_logits_s);
  if (rc != FLJSD_OK) return rc;
  JsdPlan plan;
  rc = check_jsd_workspace(BT, V, workspace, workspace_bytes, &plan);
  if (rc != FLJSD_OK) return rc;
  rc = check_device();
  if (rc != FLJSD_OK) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const double scale = reduction_scale(reduction, BT, V);
  float* row_loss = reduction == FLJSD_NONE ? loss : reinterpret_cast<float*>(ws + plan.off_row_loss);

  JsdArgs ja;
  ja.zs = logits_s;
  ja.zt = logits_t;
  ja.grad = grad_logits_s;
  ja.ld = ld;
  ja.vec_ok = ld % dtype_vec(dtype) == 0;
  ja.rows = BT;
  ja.V = V;
  ja.slice_w = plan.slices.slice_w;
  ja.S = plan.slices.S;
  ja.k2 = static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
  ja.beta = beta;
  ja.grad_scale = static_cast<float>(scale / static_cast<double>(temperature));
  ja.mode = mode_for(beta);
  ja.stats = reinterpret_cast<float4*>(ws + plan.off_stats);
  ja.lg = reinterpret_cast<float2*>(ws + plan.off_lg);
  ja.peak = reinterpret_cast<float4*>(ws + plan.off_peak);
  ja.ref = reinterpret_cast<float*>(ws + plan.off_ref);
  ja.row_loss = row_loss;
  rc = run_jsd_passes(ja, dtype, grad_logits_s != nullptr, V, dtype_size(dtype), s);
  if (rc != FLJSD_OK) return rc;
  if (reduction != FLJSD_NONE) {
    hipError_t e = timed(s, FLJSD_KCLASS_LOSS_REDUCE, 0.0, 4.0 * BT,
                         [&] { return launch_loss_reduce(row_loss, BT, static_cast<float>(scale), loss, s); });
    if (e != hipSuccess) return fail_hip(e, "launch loss reduce");
  }
  return FLJSD_OK;
}

}  // namespace
}  // namespace fljsd

// ---- scratch of the no-allocation entry point -------------------------------
// One file-scope device array per GPU (each device that loads the library
// holds its own copy until the process ends). In host code `scratch` names a
// host-side stand-in, never the device memory: the device address is looked
// up once per device with hipGetSymbolAddress and only that address is used.
// The loss passes write every byte they later read (row statistics, per-slice
// partial sums, row losses), so nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[FLJSD_NOALLOC_SCRATCH_BYTES];

namespace fljsd {
namespace {

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FLJSD_EDEVICE, "device index out of range");
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
      if (p == nullptr) return fail(FLJSD_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FLJSD_OK;
}

}  // namespace
}  // namespace fljsd

FLJSD_EXPORT int fljsd_generalized_jsd(const void* logits_s, const void* logits_t, int64_t BT,
                                       int64_t V, int64_t ld, int dtype, float beta,
                                       float temperature, int reduction, float* loss,
                                       void* grad_logits_s, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  clear_last_error();
  return generalized_jsd_impl(logits_s, logits_t, BT, V, ld, dtype, beta, temperature, reduction,
                              loss, grad_logits_s, workspace, workspace_bytes, stream);
}

FLJSD_EXPORT int fljsd_generalized_jsd_noalloc(const void* logits_s, const void* logits_t,
                                               int64_t BT, int64_t V, int64_t ld, int dtype,
                                               float beta, float temperature, int reduction,
                                               float* loss, void* grad_logits_s, void* stream) {
  clear_last_error();
  // Arguments and the scratch bound are checked before any HIP call.
  int rc = check_generalized_jsd_args(logits_s, logits_t, BT, V, ld, dtype, beta, temperature,
                                      reduction, loss, grad_logits_s);
  if (rc != FLJSD_OK) return rc;
  rc = check_noalloc_scratch(BT, V, FLJSD_NOALLOC_SCRATCH_BYTES);
  if (rc != FLJSD_OK) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != FLJSD_OK) return rc;
  return generalized_jsd_impl(logits_s, logits_t, BT, V, ld, dtype, beta, temperature, reduction,
                              loss, grad_logits_s, ws, FLJSD_NOALLOC_SCRATCH_BYTES, stream);
}

namespace fljsd {
namespace {

// Shared by the two one-pass losses: checks, planning and the launch
// sequence (element pass, per-row merge, scalar reduction).
template <class Launch>
int run_elem_loss(const void* a_ptr, const void* b_ptr, int64_t BT, int64_t V, int64_t ld,
                  int dtype, int reduction, float* loss, void* grad, bool elementwise_none,
                  bool check_beta, float beta, int mode, void* workspace, size_t workspace_bytes,
                  void* stream, int kclass, Launch&& launch) {
  JsdPlan plan;
  int rc = check_elem_loss(a_ptr, b_ptr, BT, V, ld, dtype, reduction, check_beta, beta, loss, grad,
                           workspace, workspace_bytes, &plan);
  if (rc != FLJSD_OK) return rc;
  rc = check_device();
  if (rc != FLJSD_OK) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const double scale = reduction_scale(reduction, BT, V);
  const bool none = reduction == FLJSD_NONE;
  ElemArgs ea;
  ea.a = a_ptr;
  ea.b = b_ptr;
  ea.grad = grad;
  ea.elem_loss = (none && elementwise_none) ? loss : nullptr;
  ea.ld = ld;
  ea.vec_ok = ld % dtype_vec(dtype) == 0;
  ea.rows = BT;
  ea.V = V;
  ea.slice_w = plan.slices.slice_w;
  ea.S = plan.slices.S;
  ea.beta = beta;
  ea.grad_scale = static_cast<float>(scale);
  ea.mode = mode;
  ea.lg = reinterpret_cast<float2*>(ws + plan.off_lg);
  const double bytes = static_cast<double>(BT) * V * dtype_size(dtype) * (grad ? 3 : 2);
  hipError_t e = timed(s, kclass, 0.0, bytes, [&] { return launch(ea, dtype, s); });
  if (e != hipSuccess) return fail_hip(e, "launch loss kernel");
  if (none && elementwise_none) return FLJSD_OK;
  // Per-row sums of the slice partials, then the scalar.
  JsdArgs ja;
  ja.rows = BT;
  ja.S = plan.slices.S;
  ja.lg = ea.lg;
  ja.row_loss = none ? loss : reinterpret_cast<float*>(ws + plan.off_row_loss);
  e = launch_jsd_row_loss(ja, s);
  if (e != hipSuccess) return fail_hip(e, "launch row loss");
  if (!none) {
    e = timed(s, FLJSD_KCLASS_LOSS_REDUCE, 0.0, 4.0 * BT, [&] {
      return launch_loss_reduce(ja.row_loss, BT, static_cast<float>(scale), loss, s);
    });
    if (e != hipSuccess) return fail_hip(e, "launch loss reduce");
  }
  return FLJSD_OK;
}

}  // namespace
}  // namespace fljsd

FLJSD_EXPORT int fljsd_jsd_logprob(const void* logq_s, const void* logp_t, int64_t BT, int64_t V,
                                   int64_t ld, int dtype, float beta, int reduction, float* loss,
                                   void* grad_logq_s, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  clear_last_error();
  return run_elem_loss(logq_s, logp_t, BT, V, ld, dtype, reduction, loss, grad_logq_s, false,
                       true, beta, mode_for(beta), workspace, workspace_bytes, stream,
                       FLJSD_KCLASS_ELEM_LOSS, launch_logprob_jsd);
}

FLJSD_EXPORT int fljsd_tvd(const void* p, const void* q, int64_t BT, int64_t V, int64_t ld,
                           int dtype, int reduction, float* loss, void* grad_p, void* workspace,
                           size_t workspace_bytes, void* stream) {
  clear_last_error();
  return run_elem_loss(p, q, BT, V, ld, dtype, reduction, loss, grad_p, true, false, 0.0f,
                       kModeGeneralized, workspace, workspace_bytes, stream,
                       FLJSD_KCLASS_ELEM_LOSS, launch_tvd);
}

FLJSD_EXPORT int fljsd_flce_forward_backward(const void* X, const void* W, const int64_t* labels,
                                             int64_t BT, int64_t H, int64_t V, int dtype,
                                             int64_t ignore_index, float label_smoothing,
                                             int reduction, int num_chunks, float* loss,
                                             void* grad_X, void* grad_W, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  return fljsd_flce_forward_backward_ex(X, W, labels, BT, H, V, dtype, ignore_index,
                                        label_smoothing, reduction, num_chunks, loss, grad_X,
                                        grad_W, dtype, 0u, workspace, workspace_bytes, stream);
}

FLJSD_EXPORT int fljsd_flce_forward_backward_ex(const void* X, const void* W,
                                                const int64_t* labels, int64_t BT, int64_t H,
                                                int64_t V, int dtype, int64_t ignore_index,
                                                float label_smoothing, int reduction,
                                                int num_chunks, float* loss, void* grad_X,
                                                void* grad_W, int grad_w_dtype, unsigned flags,
                                                void* workspace, size_t workspace_bytes,
                                                void* stream) {
  clear_last_error();
  CePlan plan;
  int rc = check_flce(X, W, labels, BT, H, V, dtype, label_smoothing, reduction, num_chunks, loss,
                      grad_X, grad_W, grad_w_dtype, flags, workspace, workspace_bytes, &plan);
  if (rc != FLJSD_OK) return rc;
  const bool gw_f32_acc = dtype == FLJSD_BF16 && grad_w_dtype == FLJSD_F32;
  const bool gw_add_existing = (flags & FLJSD_ACCUMULATE_GRAD_W) != 0;
  rc = check_device();
  if (rc != FLJSD_OK) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int es = dtype_size(dtype);
  char* ws = static_cast<char*>(workspace);
  void* Z = ws + plan.off_z;
  float* scale = reinterpret_cast<float*>(ws + plan.off_scale);
  float* row_loss = reduction == FLJSD_NONE ? loss : reinterpret_cast<float*>(ws + plan.off_row_loss);
  const bool write_grad = grad_X != nullptr || grad_W != nullptr;
  hipError_t e = launch_ce_scale(labels, BT, V, ignore_index, reduction, scale, s);
  if (e != hipSuccess) return fail_hip(e, "launch label count");

  CeArgs ca;
  ca.z = Z;
  ca.grad = Z;  // dZ replaces the logits in place
  ca.ld = plan.ldz;
  ca.vec_ok = true;
  ca.V = V;
  ca.slice_w = plan.slices.slice_w;
  ca.S = plan.slices.S;
  ca.ignore_index = ignore_index;
  ca.eps = label_smoothing;
  ca.stats = reinterpret_cast<float4*>(ws + plan.off_stats);
  ca.zy = reinterpret_cast<float*>(ws + plan.off_zy);
  ca.scale = scale;
  const char* Xc = static_cast<const char*>(X);
  for (int64_t ci = 0; ci < plan.n_chunks; ++ci) {
    const int64_t r0 = ci * plan.C;
    const int64_t rows = std::min(plan.C, BT - r0);
    // W^T for grad_input, written once, by the first chunk's product.
    void* wt = (grad_X && plan.w_transposed) ? ws + plan.off_wt : nullptr;
    rc = run_logits_gemm(dtype, Xc + r0 * H * es, W, Z, rows, V, H, plan.ldz, s, nullptr, 0, 0.f,
                         ci == 0 ? wt : nullptr, plan.ldz);
    if (rc != FLJSD_OK) return rc;
    ca.rows = rows;
    ca.labels = labels + r0;
    ca.row_loss = row_loss + r0;
    const double row_bytes = static_cast<double>(rows) * V * es;
    e = timed(s, FLJSD_KCLASS_CE_STATS, 0.0, row_bytes, [&] { return launch_ce_stats(ca, dtype, s); });
    if (e != hipSuccess) return fail_hip(e, "launch ce_stats");
    const bool tiled = grad_W && plan.transposed_grad_w;
    e = timed(s, FLJSD_KCLASS_CE_GRAD, 0.0, tiled ? 3 * row_bytes : (write_grad ? 2 * row_bytes : 0.0), [&] {
      return tiled ? launch_ce_grad_transposed(ca, ws + plan.off_zt, plan.ldt, s)
                   : launch_ce_grad(ca, dtype, write_grad, s);
    });
    if (e != hipSuccess) return fail_hip(e, "launch ce_grad");
    if (grad_X) {
      rc = run_grad_input(dtype, Z, plan.ldz, W, rows, H, V,
                          static_cast<char*>(grad_X) + r0 * H * es, plan.splitk,
                          plan.k_per_split, ws + plan.off_partial, s, wt, plan.ldz);
      if (rc != FLJSD_OK) return rc;
    }
    if (grad_W) {
      // As in the JSD pass: chunk 0 overwrites unless asked to add; an fp32
      // grad_W takes the bf16 products unrounded (PR #1429, Details).
      const bool add = ci > 0 || gw_add_existing;
      const int epi = gw_f32_acc ? (add ? kEpiAccumulateF32 : kEpiPartialF32)
                                 : (add ? kEpiAccumulate : kEpiStore);
      rc = run_grad_weight(dtype, Z, plan.ldz, Xc + r0 * H * es, rows, H, V, grad_W,
                           plan.transposed_grad_w, ws + plan.off_zt, ws + plan.off_xt, plan.ldt,
                           epi, s, /*dz_transposed=*/true);
      if (rc != FLJSD_OK) return rc;
    }
  }
  if (reduction != FLJSD_NONE) {
    e = timed(s, FLJSD_KCLASS_LOSS_REDUCE, 0.0, 4.0 * BT,
              [&] { return launch_loss_reduce_dev(row_loss, BT, scale, loss, s); });
    if (e != hipSuccess) return fail_hip(e, "launch loss reduce");
  }
  return FLJSD_OK;
}
