// Test-only recording launcher for the CPU build of the host logic.
//
// Linked with ring.cpp and plan.cpp into _build/libkvc_hostcheck.so.  Instead
// of launching kernels it records each request so the Python tests can check
// the ring's bookkeeping (which slot each write targets, the logical segment
// table handed to attention) without a GPU.  It can also be told to fail the
// next launch, to check that a failed call leaves the ring unchanged.
#include <cstdint>
#include <cstring>
#include <vector>

#include "e4m3_rule.hpp"
#include "kvc_internal.hpp"

namespace {

struct Record {
  int32_t kind;       // 0 cache write, 1 attention (dst_k: workspace), 2 edit mask
                      // (mask: rows = tokens, pitch = channels, nseg = keep,
                      // scale = tau, src_k/src_v = z_src/z_edit,
                      // dst_k/dst_vt = rows/count)
  int32_t rows;       // write: rows; attention: n
  int32_t pitch;      // write: pitch
  int32_t nseg;       // attention
  uint64_t dst_k;     // write: K destination
  uint64_t dst_vt;    // write: Vt destination
  uint64_t src_k;     // write: caller k; attention: q
  uint64_t src_v;     // write: caller v; attention: o
  uint64_t seg_k[kvc::kMaxSegments];
  int32_t seg_rows[kvc::kMaxSegments];
  int32_t seg_pitch[kvc::kMaxSegments];
  float scale;
  int32_t kv_dtype;
  uint64_t k_scale;   // write (fp8)
  uint64_t stream;
  uint64_t qrows;     // attention: active-row map (0: all rows)
  uint64_t qcount;    // attention: active-row count
  uint64_t rope;      // write: K rotation table; attention: q rotation table
  uint32_t epoch;     // attention: the call's epoch
  int32_t ws_ready;   // attention: workspace already zeroed by an earlier call
};

std::vector<Record> g_log;
kvc_status g_fail = KVC_OK;

kvc_status take_failure() {
  kvc_status s = g_fail;
  g_fail = KVC_OK;
  return s;
}

}  // namespace

namespace kvc {

kvc_status launch_cache_write(const CacheWriteDesc& d, void* stream) {
  if (kvc_status s = take_failure()) return s;
  Record r;
  std::memset(&r, 0, sizeof(r));
  r.kind = 0;
  r.rows = d.rows;
  r.pitch = d.pitch;
  r.dst_k = reinterpret_cast<uint64_t>(d.k_dst);
  r.dst_vt = reinterpret_cast<uint64_t>(d.vt_dst);
  r.src_k = reinterpret_cast<uint64_t>(d.k);
  r.src_v = reinterpret_cast<uint64_t>(d.v);
  r.kv_dtype = d.kv_dtype;
  r.k_scale = reinterpret_cast<uint64_t>(d.k_scale);
  r.stream = reinterpret_cast<uint64_t>(stream);
  r.rope = reinterpret_cast<uint64_t>(d.rope);
  g_log.push_back(r);
  return KVC_OK;
}

kvc_status launch_attention(const AttnDesc& d, void* stream) {
  if (kvc_status s = take_failure()) return s;
  Record r;
  std::memset(&r, 0, sizeof(r));
  r.kind = 1;
  r.rows = d.n;
  r.nseg = d.nseg;
  r.src_k = reinterpret_cast<uint64_t>(d.q);
  r.src_v = reinterpret_cast<uint64_t>(d.o);
  for (int s = 0; s < d.nseg; ++s) {
    r.seg_k[s] = reinterpret_cast<uint64_t>(d.seg[s].k);
    r.seg_rows[s] = d.seg[s].rows;
    r.seg_pitch[s] = d.seg[s].pitch;
  }
  r.scale = d.scale;
  r.kv_dtype = d.kv_dtype;
  r.stream = reinterpret_cast<uint64_t>(stream);
  r.qrows = reinterpret_cast<uint64_t>(d.qrows);
  r.qcount = reinterpret_cast<uint64_t>(d.qcount);
  r.rope = reinterpret_cast<uint64_t>(d.qrope);
  r.epoch = d.epoch;
  r.ws_ready = d.workspace_ready ? 1 : 0;
  r.dst_k = reinterpret_cast<uint64_t>(d.workspace);
  g_log.push_back(r);
  return KVC_OK;
}

kvc_status launch_edit_mask(const EditMaskDesc& d, void* stream) {
  if (kvc_status s = take_failure()) return s;
  Record r;
  std::memset(&r, 0, sizeof(r));
  r.kind = 2;
  r.rows = d.tokens;
  r.pitch = d.channels;
  r.nseg = d.keep;
  r.scale = d.tau;
  r.src_k = reinterpret_cast<uint64_t>(d.z_src);
  r.src_v = reinterpret_cast<uint64_t>(d.z_edit);
  r.dst_k = reinterpret_cast<uint64_t>(d.rows);
  r.dst_vt = reinterpret_cast<uint64_t>(d.count);
  r.stream = reinterpret_cast<uint64_t>(stream);
  g_log.push_back(r);
  return KVC_OK;
}

// The static workspace of chunk_attn_fwd_noalloc: a fake device address
// (the host code never dereferences it), epochs counted as on the device.
namespace {
uint32_t g_static_epoch = 0;
bool g_static_ready = false;
}  // namespace

kvc_status static_workspace(size_t need, StaticWork& w) {
  if (need > KVC_NOALLOC_SCRATCH_BYTES) return KVC_E_SCRATCH;
  w.ptr = reinterpret_cast<void*>(0x7E0000000000ull);
  w.bytes = KVC_NOALLOC_SCRATCH_BYTES;
  w.ready = g_static_ready;
  g_static_epoch = g_static_epoch + 1 == 0 ? 1 : g_static_epoch + 1;
  w.epoch = g_static_epoch;
  w.device = 0;
  return KVC_OK;
}

void static_workspace_launched(const StaticWork&) { g_static_ready = true; }

}  // namespace kvc

extern "C" {

int32_t kvcfake_record_size() { return static_cast<int32_t>(sizeof(Record)); }
int32_t kvcfake_count() { return static_cast<int32_t>(g_log.size()); }
void kvcfake_reset() { g_log.clear(); g_fail = KVC_OK; }
void kvcfake_fail_next(int32_t status) { g_fail = status; }
int32_t kvcfake_get(int32_t i, void* out) {
  if (i < 0 || i >= static_cast<int32_t>(g_log.size())) return -1;
  std::memcpy(out, &g_log[i], sizeof(Record));
  return 0;
}

// The C statement of the E4M3 rule (e4m3_rule.hpp), for CPU tests against
// the oracle.
void kvcfake_e4m3_encode(const float* x, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = kvc::e4m3_from_float(x[i]);
}

}  // extern "C"
