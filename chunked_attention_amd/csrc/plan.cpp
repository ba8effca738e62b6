// Host-side planning shared by the device build and the CPU test build:
// device workspace of an attention call.
#include "kvc_internal.hpp"

namespace kvc {

// Workspace of the attention kernel: per row two counters (pieces arrived,
// partials written), then per persistent workgroup two partial slots, each
// holding the reference max and two sums (of the bf16-rounded and of the
// exact probabilities) of its queries and the unnormalised fp32 output
// [kAttnRowQueries][d].
size_t attention_workspace_bytes(int heads, int head_dim, int n, int kv_dtype) {
  (void)kv_dtype;
  const size_t nrows = static_cast<size_t>(heads) *
                       ((n + kAttnRowQueries - 1) / kAttnRowQueries);
  const size_t counters = align_up(sizeof(unsigned) * 2 * nrows, 256);
  const size_t ml = align_up(sizeof(float) * 2 * kAttnMaxWg * 3 * kAttnRowQueries, 256);
  const size_t po = sizeof(float) * 2 * static_cast<size_t>(kAttnMaxWg) * kAttnRowQueries *
                    head_dim;
  return counters + ml + po;
}

}  // namespace kvc
