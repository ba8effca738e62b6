// Host-side planning shared by the device build and the CPU test build:
// device workspace of an attention call.
#include "kvc_internal.hpp"

namespace kvc {

WorkLayout attention_workspace_layout(int heads, int head_dim, int n) {
  WorkLayout L;
  L.rows = heads * ((n + kAttnRowQueries - 1) / kAttnRowQueries);
  const size_t slots = 2 * static_cast<size_t>(kAttnMaxWg);
  L.arrive_off = 0;
  L.tags_off = align_up(sizeof(unsigned long long) * L.rows, 256);
  L.ml_off = L.tags_off + align_up(sizeof(unsigned) * slots, 256);
  L.po_off = L.ml_off + align_up(sizeof(float) * slots * 2 * kAttnRowQueries, 256);
  L.total = L.po_off + sizeof(float) * slots * kAttnRowQueries * static_cast<size_t>(head_dim);
  L.zero_words = static_cast<int>(L.ml_off / sizeof(unsigned));
  return L;
}

size_t attention_workspace_bytes(int heads, int head_dim, int n, int kv_dtype) {
  (void)kv_dtype;
  return attention_workspace_layout(heads, head_dim, n).total;
}

}  // namespace kvc
