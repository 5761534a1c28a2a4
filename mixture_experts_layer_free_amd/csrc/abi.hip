// Host-side parts of the C ABI: workspace sizes, status strings and the
// per-device compute-unit count.
#include <atomic>

#include "aux.h"
#include "moe_common.h"

size_t moe_permute_workspace(int64_t T, int k, int E);
size_t moe_ffn_workspace(int G);
size_t moe_backward_workspace(int64_t T, int k, int E, int64_t d, int64_t f);
size_t moe_backward_shared_workspace(int64_t T, int64_t d, int64_t fs);

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0 = not yet queried
}  // namespace

int moe_num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

extern "C" size_t moe_workspace_size(int which, int64_t T, int k, int E, int64_t d, int64_t f) {
  if (T < 1 || k < 1 || E < 1) return 0;
  switch (which) {
    case MOE_CALL_ROUTE:
      return 0;
    case MOE_CALL_PERMUTE:
      return moe_permute_workspace(T, k, E);
    case MOE_CALL_GROUPED_FFN:
      return moe_ffn_workspace(E);
    case MOE_CALL_BACKWARD:
      return moe_backward_workspace(T, k, E, d, f);
    case MOE_CALL_AUX_LOSS:
      return moe_aux_workspace(T, E);
    case MOE_CALL_BACKWARD_SHARED:
      return moe_backward_shared_workspace(T, d, f);
    default:
      return 0;
  }
}

extern "C" const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ENOTSUP: return "shape or option not supported";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}
