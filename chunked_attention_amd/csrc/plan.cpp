// Host-side planning shared by the device build and the CPU test build:
// how much device workspace an attention call may use.
#include "kvc_internal.hpp"

namespace kvc {

size_t attention_workspace_bytes(int heads, int head_dim, int n, int kv_dtype) {
  (void)heads;
  (void)head_dim;
  (void)n;
  (void)kv_dtype;
  return 0;
}

}  // namespace kvc
