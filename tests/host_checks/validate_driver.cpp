// Host-only driver of the library's argument checks and planning arithmetic,
// built by the test suite with a host compiler under AddressSanitizer and
// UndefinedBehaviorSanitizer (no HIP, no GPU). One case per input line; one
// result per output line.
//
//   fb    X_s W_s X_t W_t BT H_s H_t V dtype beta T reduction nc loss gX gW gw_dtype flags ws ws_bytes
//   jsd   zs zt BT V ld dtype beta T reduction loss grad ws ws_bytes
//   noalloc zs zt BT V ld dtype beta T reduction loss grad
//   elem  kind(0 = log-probability JSD, 1 = TVD) a b BT V ld dtype beta reduction loss grad ws ws_bytes
//   flce  X W labels BT H V dtype ls reduction nc loss gX gW gw_dtype flags ws ws_bytes
//   ws    BT H_s H_t V dtype nc          (fljsd_workspace_size)
//   gws   BT V dtype                     (fljsd_generalized_jsd_workspace_size)
//   plan  BT H_s H_t V dtype budget      (fljsd_plan_num_chunks)
//   flcews BT H V dtype nc               (fljsd_flce_workspace_size)
//   flceplan BT H V dtype budget         (fljsd_flce_plan_num_chunks)
// Pointers are integers (0 = NULL; never dereferenced); floats accept nan/inf.
#include "fljsd.h"
#include "plan.h"
#include "validate.h"

#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>

namespace {

struct Reader {
  std::istringstream in;
  explicit Reader(const std::string& s) : in(s) {}
  std::string word() {
    std::string w;
    in >> w;
    return w;
  }
  const void* ptr() { return reinterpret_cast<const void*>(static_cast<uintptr_t>(std::strtoull(word().c_str(), nullptr, 0))); }
  int64_t i64() { return std::strtoll(word().c_str(), nullptr, 0); }
  uint64_t u64() { return std::strtoull(word().c_str(), nullptr, 0); }
  int i32() { return static_cast<int>(i64()); }
  float f32() { return std::strtof(word().c_str(), nullptr); }
};

}  // namespace

int main() {
  using namespace fljsd;
  std::string line;
  while (std::getline(std::cin, line)) {
    if (line.empty()) continue;
    Reader r(line);
    const std::string op = r.word();
    long long out = 0;
    if (op == "fb") {
      const void *Xs = r.ptr(), *Ws = r.ptr(), *Xt = r.ptr(), *Wt = r.ptr();
      const int64_t BT = r.i64(), Hs = r.i64(), Ht = r.i64(), V = r.i64();
      const int dtype = r.i32();
      const float beta = r.f32(), T = r.f32();
      const int red = r.i32(), nc = r.i32();
      const float* loss = static_cast<const float*>(r.ptr());
      const void *gX = r.ptr(), *gW = r.ptr();
      const int gwd = r.i32();
      const unsigned flags = static_cast<unsigned>(r.u64());
      const void* ws = r.ptr();
      const size_t wsb = r.u64();
      ChunkPlan plan;
      out = check_forward_backward(Xs, Ws, Xt, Wt, BT, Hs, Ht, V, dtype, beta, T, red, nc, loss, gX,
                                   gW, gwd, flags, ws, wsb, &plan);
    } else if (op == "jsd" || op == "noalloc") {
      const void *zs = r.ptr(), *zt = r.ptr();
      const int64_t BT = r.i64(), V = r.i64(), ld = r.i64();
      const int dtype = r.i32();
      const float beta = r.f32(), T = r.f32();
      const int red = r.i32();
      const float* loss = static_cast<const float*>(r.ptr());
      const void* grad = r.ptr();
      out = check_generalized_jsd_args(zs, zt, BT, V, ld, dtype, beta, T, red, loss, grad);
      if (out == FLJSD_OK && op == "jsd") {
        const void* ws = r.ptr();
        const size_t wsb = r.u64();
        JsdPlan plan;
        out = check_jsd_workspace(BT, V, ws, wsb, &plan);
      } else if (out == FLJSD_OK) {
        out = check_noalloc_scratch(BT, V, FLJSD_NOALLOC_SCRATCH_BYTES);
      }
    } else if (op == "elem") {
      const int kind = r.i32();
      const void *a = r.ptr(), *b = r.ptr();
      const int64_t BT = r.i64(), V = r.i64(), ld = r.i64();
      const int dtype = r.i32();
      const float beta = r.f32();
      const int red = r.i32();
      const float* loss = static_cast<const float*>(r.ptr());
      const void* grad = r.ptr();
      const void* ws = r.ptr();
      const size_t wsb = r.u64();
      JsdPlan plan;
      out = check_elem_loss(a, b, BT, V, ld, dtype, red, kind == 0, beta, loss, grad, ws, wsb, &plan);
    } else if (op == "flce") {
      const void *X = r.ptr(), *W = r.ptr();
      const int64_t* labels = static_cast<const int64_t*>(r.ptr());
      const int64_t BT = r.i64(), H = r.i64(), V = r.i64();
      const int dtype = r.i32();
      const float ls = r.f32();
      const int red = r.i32(), nc = r.i32();
      const float* loss = static_cast<const float*>(r.ptr());
      const void *gX = r.ptr(), *gW = r.ptr();
      const int gwd = r.i32();
      const unsigned flags = static_cast<unsigned>(r.u64());
      const void* ws = r.ptr();
      const size_t wsb = r.u64();
      CePlan plan;
      out = check_flce(X, W, labels, BT, H, V, dtype, ls, red, nc, loss, gX, gW, gwd, flags, ws, wsb,
                       &plan);
    } else if (op == "ws") {
      const int64_t BT = r.i64(), Hs = r.i64(), Ht = r.i64(), V = r.i64();
      const int dtype = r.i32(), nc = r.i32();
      out = static_cast<long long>(fljsd_workspace_size(BT, Hs, Ht, V, dtype, nc));
    } else if (op == "gws") {
      const int64_t BT = r.i64(), V = r.i64();
      out = static_cast<long long>(fljsd_generalized_jsd_workspace_size(BT, V, r.i32()));
    } else if (op == "plan") {
      const int64_t BT = r.i64(), Hs = r.i64(), Ht = r.i64(), V = r.i64();
      const int dtype = r.i32();
      out = fljsd_plan_num_chunks(BT, Hs, Ht, V, dtype, r.u64());
    } else if (op == "flcews") {
      const int64_t BT = r.i64(), H = r.i64(), V = r.i64();
      const int dtype = r.i32(), nc = r.i32();
      out = static_cast<long long>(fljsd_flce_workspace_size(BT, H, V, dtype, nc));
    } else if (op == "flceplan") {
      const int64_t BT = r.i64(), H = r.i64(), V = r.i64();
      const int dtype = r.i32();
      out = fljsd_flce_plan_num_chunks(BT, H, V, dtype, r.u64());
    } else {
      std::fprintf(stderr, "unknown case: %s\n", line.c_str());
      return 2;
    }
    std::printf("%lld\n", out);
  }
  return 0;
}
