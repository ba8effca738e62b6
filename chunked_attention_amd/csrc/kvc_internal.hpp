// Internal interface between the host ring logic (ring.cpp, plain C++) and
// the device launchers (launch_*.hip).  Nothing here includes HIP headers, so
// the ring logic builds and is tested on a host without a GPU against a
// recording launcher.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/kvc.h"

namespace kvc {

constexpr int kMaxSegments = KVC_MAX_SEGMENTS;   // cond, ref, sink, W, current, source
constexpr int kTileKeys = KVC_TILE_KEYS;

// Attention work decomposition (shared by the launcher and the workspace
// sizing): a row is kAttnRowQueries queries of one head, run by one
// workgroup; at most kAttnMaxWg persistent workgroups split the rows' key
// tiles.
constexpr int kAttnRowQueries = 128;
constexpr int kAttnMaxWg = 512;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int pad_rows(int r) { return (r + kTileKeys - 1) / kTileKeys * kTileKeys; }

// One stored slot of R rows (see kvc.h for the layout).
struct SlotGeom {
  int rows = 0;        // R
  int pitch = 0;       // P, R rounded up to kTileKeys
  size_t k_off = 0;    // byte offsets from the ring base
  size_t vt_off = 0;
  size_t scale_off = 0;  // float32 [2][H]; only for fp8 rings
  size_t bytes = 0;      // total bytes of the slot
};

// Description of one cache write (condition rows or a chunk).
struct CacheWriteDesc {
  const void* k = nullptr;     // [rows][H][d] bf16, token-major
  const void* v = nullptr;
  int rows = 0;
  int pitch = 0;
  int heads = 0;
  int head_dim = 0;
  int kv_dtype = KVC_KV_BF16;
  void* k_dst = nullptr;       // [H][pitch][d]
  void* vt_dst = nullptr;      // [H][pitch/T][d][T], T = 32 (bf16) or 64 (fp8)
  float* k_scale = nullptr;    // [H] (fp8)
  float* v_scale = nullptr;    // [H] (fp8)
  float* scratch = nullptr;    // fp8: float32 [2][H][pitch/kTileKeys] partial amax
  const float* rope = nullptr; // optional rotation of K: float32 [rows][d/2][(cos, sin)]
};

// One logical segment of the visible KV, in device terms.
struct AttnSegment {
  const void* k = nullptr;      // [H][pitch][d]
  const void* vt = nullptr;     // [H][pitch/T][d][T], T = 32 (bf16) or 64 (fp8)
  const float* k_scale = nullptr;
  const float* v_scale = nullptr;
  int rows = 0;
  int pitch = 0;
};

struct AttnDesc {
  const void* q = nullptr;      // [n][H][d] bf16
  void* o = nullptr;            // [n][H][d] bf16
  float* lse = nullptr;         // [H][n] or null
  // active-row calls: only rows qrows[0 .. *qcount) of q / o / lse are
  // computed (device memory; *qcount is clamped to [0, n]); null: all rows
  const int32_t* qrows = nullptr;
  const int32_t* qcount = nullptr;
  const float* qrope = nullptr;  // optional rotation of q: float32 [n][d/2][(cos, sin)]
  int n = 0;
  int heads = 0;
  int head_dim = 0;
  int kv_dtype = KVC_KV_BF16;
  float scale = 0.f;            // softmax scale (natural-log units)
  int nseg = 0;
  AttnSegment seg[kMaxSegments];
  void* workspace = nullptr;    // device scratch for split partials
  size_t workspace_bytes = 0;
  bool workspace_ready = false; // arrival words and tags in the workspace already zeroed
  uint32_t epoch = 1;           // nonzero, different from the previous call's on this workspace
};

// LiveEdit active-row mask (validated by the caller).
struct EditMaskDesc {
  const void* z_src = nullptr;  // [tokens][channels] bf16
  const void* z_edit = nullptr;
  int tokens = 0;               // 1..KVC_MAX_MASK_TOKENS
  int channels = 0;
  float tau = 0.f;              // threshold mode (keep < 0)
  int keep = -1;                // top-k mode (keep >= 0)
  int32_t* rows = nullptr;      // [tokens]
  int32_t* count = nullptr;     // [1]
};

// Launchers.  Return KVC_OK or KVC_E_DEVICE / KVC_E_UNSUPPORTED.  The device
// implementation lives in the HIP sources; tests link a recording fake.
kvc_status launch_cache_write(const CacheWriteDesc& d, void* stream);
kvc_status launch_attention(const AttnDesc& d, void* stream);
kvc_status launch_edit_mask(const EditMaskDesc& d, void* stream);

// Attention workspace of a ring whose calls have n queries (byte offsets
// from its start, each part 256-byte aligned):
//   arrive  uint64 [rows]: per 128-query row, (epoch << 32) | pieces arrived
//   tags    uint32 [2 * kAttnMaxWg]: per partial slot, the epoch of the call
//           that last stored it
//   ml      float32 [2 * kAttnMaxWg][4 waves][2][32]: partial reference and sum
//   po      float32 [2 * kAttnMaxWg][kAttnRowQueries * head_dim]: partial O
// The arrival words and tags are zero before a ring's first call; after that
// the epoch of each call tells its own words from stale ones.
struct WorkLayout {
  size_t arrive_off = 0, tags_off = 0, ml_off = 0, po_off = 0, total = 0;
  int rows = 0;            // 128-query rows
  int zero_words = 0;      // 32-bit words from the start to zero before first use
};
WorkLayout attention_workspace_layout(int heads, int head_dim, int n);
size_t attention_workspace_bytes(int heads, int head_dim, int n, int kv_dtype);

// The attention workspace held in the library's static device array
// (chunk_attn_fwd_noalloc), on the current device.
struct StaticWork {
  void* ptr = nullptr;      // device address of the array on this device
  size_t bytes = 0;
  bool ready = false;       // arrival words and tags already zeroed on this device
  uint32_t epoch = 0;       // this call's epoch on this device (nonzero)
  int device = -1;
};
// Fills `w` for a call needing `need` bytes: KVC_E_SCRATCH if need exceeds
// KVC_NOALLOC_SCRATCH_BYTES, KVC_E_DEVICE if the runtime fails.  Allocates
// nothing.
kvc_status static_workspace(size_t need, StaticWork& w);
// after a successful launch with `w`: its zeroing has been enqueued
void static_workspace_launched(const StaticWork& w);

}  // namespace kvc
