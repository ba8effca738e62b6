// Ring-buffer KV cache and the C ABI (host side, plain C++17).
//
// The cache holds the condition rows, the reference rows, the global sink
// (chunk 0), a sliding window of the W most recent committed chunks, one
// staging slot for the chunk being generated and one slot for that chunk's
// source tokens: W + 2 chunk slots recycled in place, so memory and
// per-chunk work stay bounded for an open-ended stream (discuss.pytorch.kr
// "JoyAI-Video-Edit 소개", real-time deployment section; ta-paperlens section
// 5, per-chunk loop: denoise with the cache as history, then update it keeping
// only the window and the sink).
//
// Every call validates first, then launches, and only then changes state, so
// a failed call leaves the ring as it was.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>

#include "kvc_internal.hpp"

namespace kvc {
namespace {

bool config_ok(const kvc_config* c) {
  if (!c) return false;
  if (c->heads < 1 || c->heads > 4096) return false;
  if (c->head_dim != 64 && c->head_dim != 128) return false;
  if (c->chunk_tokens < 1 || c->chunk_tokens > (1 << 20)) return false;
  if (c->cond_tokens < 0 || c->cond_tokens > (1 << 20)) return false;
  if (c->ref_tokens < 0 || c->ref_tokens > (1 << 20)) return false;
  if (c->source_tokens < 0 || c->source_tokens > (1 << 20)) return false;
  if (c->window < 0 || c->window > KVC_MAX_WINDOW) return false;
  if (c->kv_dtype != KVC_KV_BF16 && c->kv_dtype != KVC_KV_FP8_E4M3) return false;
  if (!(c->softmax_scale >= 0.f) || !std::isfinite(c->softmax_scale)) return false;
  return true;
}

SlotGeom make_slot(const kvc_config& c, int rows, size_t offset) {
  SlotGeom g;
  g.rows = rows;
  g.pitch = pad_rows(rows);
  const size_t e = c.kv_dtype == KVC_KV_FP8_E4M3 ? 1 : 2;
  const size_t part = align_up(size_t(c.heads) * g.pitch * c.head_dim * e, KVC_ALIGN);
  g.k_off = offset;
  g.vt_off = offset + part;
  size_t end = g.vt_off + part;
  if (c.kv_dtype == KVC_KV_FP8_E4M3) {
    g.scale_off = end;
    end += align_up(sizeof(float) * 2 * c.heads, KVC_ALIGN);
  }
  g.bytes = end - offset;
  return g;
}

struct Layout {
  SlotGeom cond;                 // rows == 0 when m == 0
  SlotGeom ref;                  // rows == 0 when r == 0
  SlotGeom chunk[KVC_MAX_WINDOW + 2];
  SlotGeom source;               // rows == 0 when s == 0
  int n_slots = 0;
  size_t scratch_off = 0, scratch_bytes = 0;     // cache-write scratch (fp8)
  size_t work_off = 0, work_bytes = 0;           // attention workspace
  size_t total = 0;
};

Layout make_layout(const kvc_config& c) {
  Layout L;
  size_t off = 0;
  if (c.cond_tokens > 0) {
    L.cond = make_slot(c, c.cond_tokens, off);
    off += L.cond.bytes;
  }
  if (c.ref_tokens > 0) {
    L.ref = make_slot(c, c.ref_tokens, off);
    off += L.ref.bytes;
  }
  L.n_slots = c.window + 2;
  for (int i = 0; i < L.n_slots; ++i) {
    L.chunk[i] = make_slot(c, c.chunk_tokens, off);
    off += L.chunk[i].bytes;
  }
  if (c.source_tokens > 0) {
    L.source = make_slot(c, c.source_tokens, off);
    off += L.source.bytes;
  }
  if (c.kv_dtype == KVC_KV_FP8_E4M3) {
    const int maxrows = std::max(std::max(c.chunk_tokens, c.cond_tokens),
                                 std::max(c.ref_tokens, c.source_tokens));
    L.scratch_off = off;
    L.scratch_bytes = align_up(sizeof(float) * 2 * c.heads * (pad_rows(maxrows) / kTileKeys),
                               KVC_ALIGN);
    off += L.scratch_bytes;
  }
  L.work_off = off;
  L.work_bytes = align_up(attention_workspace_bytes(c.heads, c.head_dim,
                                                    c.chunk_tokens + c.source_tokens,
                                                    c.kv_dtype), KVC_ALIGN);
  off += L.work_bytes;
  L.total = off;
  return L;
}

}  // namespace
}  // namespace kvc

struct kvc_ring {
  kvc_config cfg;
  kvc::Layout L;
  unsigned char* base;
  float scale;
  // slot_chunk[i]: committed chunk id held by slot i, -1 if none
  int slot_chunk[KVC_MAX_WINDOW + 2];
  int sink_slot;          // slot of chunk 0, -1 until committed
  // committed window chunks, oldest first (sink excluded): ids and slots
  int win_id[KVC_MAX_WINDOW + 2];
  int win_slot[KVC_MAX_WINDOW + 2];
  int n_win;
  int t;                  // current chunk id (next one in phase EMPTY)
  int phase;
  int staging;            // staging slot in phase STAGED, -1 otherwise
  int current;            // slot of the current chunk (STAGED or COMMITTED)
  int cond_valid;
  int ref_valid;
  int work_ready;         // attention workspace arrival words and tags zeroed
  uint32_t epoch;         // epoch of the last attention call (0: none yet)
};

namespace kvc {
namespace {

int free_slot(const kvc_ring* r) {
  for (int i = 0; i < r->L.n_slots; ++i) {
    if (r->slot_chunk[i] < 0 && i != r->staging) return i;
  }
  return -1;
}

CacheWriteDesc write_desc(const kvc_ring* r, const SlotGeom& g, const void* k, const void* v,
                          const float* rope) {
  CacheWriteDesc d;
  d.rope = rope;
  d.k = k;
  d.v = v;
  d.rows = g.rows;
  d.pitch = g.pitch;
  d.heads = r->cfg.heads;
  d.head_dim = r->cfg.head_dim;
  d.kv_dtype = r->cfg.kv_dtype;
  d.k_dst = r->base + g.k_off;
  d.vt_dst = r->base + g.vt_off;
  if (r->cfg.kv_dtype == KVC_KV_FP8_E4M3) {
    d.k_scale = reinterpret_cast<float*>(r->base + g.scale_off);
    d.v_scale = d.k_scale + r->cfg.heads;
    d.scratch = reinterpret_cast<float*>(r->base + r->L.scratch_off);
  }
  return d;
}

AttnSegment seg_of(const kvc_ring* r, const SlotGeom& g) {
  AttnSegment s;
  s.k = r->base + g.k_off;
  s.vt = r->base + g.vt_off;
  if (r->cfg.kv_dtype == KVC_KV_FP8_E4M3) {
    s.k_scale = reinterpret_cast<const float*>(r->base + g.scale_off);
    s.v_scale = s.k_scale + r->cfg.heads;
  }
  s.rows = g.rows;
  s.pitch = g.pitch;
  return s;
}

// Logical segment table for an attention call now: [cond ; ref ; sink ;
// window chunks max(1,t-W)..t-1 oldest first ; current ; source].  Returns
// the count, or -1 when no call is possible.
int segment_table(const kvc_ring* r, kvc_segment* info, AttnSegment* dev) {
  if (r->phase == KVC_PHASE_EMPTY) return -1;
  if (r->cfg.cond_tokens > 0 && !r->cond_valid) return -1;
  if (r->cfg.ref_tokens > 0 && !r->ref_valid) return -1;
  int n = 0;
  if (r->cfg.cond_tokens > 0) {
    if (info) info[n] = kvc_segment{-1, -1, r->cfg.cond_tokens, 0};
    if (dev) dev[n] = seg_of(r, r->L.cond);
    ++n;
  }
  if (r->cfg.ref_tokens > 0) {
    if (info) info[n] = kvc_segment{-1, -3, r->cfg.ref_tokens, 4};
    if (dev) dev[n] = seg_of(r, r->L.ref);
    ++n;
  }
  const int t = r->t;
  if (t >= 1) {
    if (r->sink_slot < 0) return -1;
    if (info) info[n] = kvc_segment{0, r->sink_slot, r->cfg.chunk_tokens, 1};
    if (dev) dev[n] = seg_of(r, r->L.chunk[r->sink_slot]);
    ++n;
  }
  const int lo = t - r->cfg.window > 1 ? t - r->cfg.window : 1;
  int expect = lo;
  for (int i = 0; i < r->n_win; ++i) {
    const int id = r->win_id[i];
    if (id < lo || id >= t) continue;
    if (id != expect) return -1;          // a visible chunk is missing
    ++expect;
    if (info) info[n] = kvc_segment{id, r->win_slot[i], r->cfg.chunk_tokens, 2};
    if (dev) dev[n] = seg_of(r, r->L.chunk[r->win_slot[i]]);
    ++n;
  }
  if (expect != t && t >= 1) return -1;
  if (info) info[n] = kvc_segment{t, r->current, r->cfg.chunk_tokens, 3};
  if (dev) dev[n] = seg_of(r, r->L.chunk[r->current]);
  ++n;
  if (r->cfg.source_tokens > 0) {
    if (info) info[n] = kvc_segment{t, -4, r->cfg.source_tokens, 5};
    if (dev) dev[n] = seg_of(r, r->L.source);
    ++n;
  }
  return n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

kvc_status attention_call(kvc_ring* r, const void* q, void* o, float* lse, const float* rope,
                          const int32_t* rows, const int32_t* count, void* stream,
                          bool static_work = false) {
  if (!r || !q || !o || !aligned16(q) || !aligned16(o) || q == o) return KVC_E_INVAL;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return KVC_E_INVAL;
  if (rope && !aligned16(rope)) return KVC_E_INVAL;
  AttnDesc d;
  d.qrows = rows;
  d.qcount = count;
  d.qrope = rope;
  d.nseg = segment_table(r, nullptr, d.seg);
  if (d.nseg < 0) return KVC_E_STATE;
  d.q = q;
  d.o = o;
  d.lse = lse;
  d.n = r->cfg.chunk_tokens + r->cfg.source_tokens;
  d.heads = r->cfg.heads;
  d.head_dim = r->cfg.head_dim;
  d.kv_dtype = r->cfg.kv_dtype;
  d.scale = r->scale;
  if (static_work) {
    // the library's static device array on the current device (its own
    // epochs: it is shared by every ring on the device)
    StaticWork sw;
    const kvc_status ws = static_workspace(
        attention_workspace_bytes(d.heads, d.head_dim, d.n, d.kv_dtype), sw);
    if (ws != KVC_OK) return ws;
    d.workspace = sw.ptr;
    d.workspace_bytes = sw.bytes;
    d.workspace_ready = sw.ready;
    d.epoch = sw.epoch;
    const kvc_status s = launch_attention(d, stream);
    if (s == KVC_OK) static_workspace_launched(sw);
    return s;
  }
  d.workspace = r->base + r->L.work_off;
  d.workspace_bytes = r->L.work_bytes;
  d.workspace_ready = r->work_ready != 0;
  // every call gets a new nonzero epoch: the kernel tells this call's
  // arrival words and partial tags in the workspace from earlier calls' by it
  d.epoch = r->epoch + 1 == 0 ? 1 : r->epoch + 1;
  kvc_status s = launch_attention(d, stream);
  if (s == KVC_OK) {
    r->work_ready = 1;
    r->epoch = d.epoch;
  }
  return s;
}

kvc_status append(kvc_ring* r, int32_t kind, const void* k, const void* v, const float* rope,
                  void* stream) {
  if (!r || !k || !v || !aligned16(k) || !aligned16(v)) return KVC_E_INVAL;
  if (rope && !aligned16(rope)) return KVC_E_INVAL;
  if (kind == KVC_COND) {
    if (r->cfg.cond_tokens <= 0) return KVC_E_INVAL;
    kvc_status s = launch_cache_write(write_desc(r, r->L.cond, k, v, rope), stream);
    if (s != KVC_OK) return s;
    r->cond_valid = 1;
    return KVC_OK;
  }
  if (kind == KVC_REF) {
    if (r->cfg.ref_tokens <= 0) return KVC_E_INVAL;
    kvc_status s = launch_cache_write(write_desc(r, r->L.ref, k, v, rope), stream);
    if (s != KVC_OK) return s;
    r->ref_valid = 1;
    return KVC_OK;
  }
  if (kind != KVC_STAGE && kind != KVC_COMMIT) return KVC_E_INVAL;
  if (r->phase == KVC_PHASE_COMMITTED) return KVC_E_STATE;
  int slot = r->phase == KVC_PHASE_STAGED ? r->staging : free_slot(r);
  if (slot < 0) return KVC_E_STATE;
  kvc_status s = launch_cache_write(write_desc(r, r->L.chunk[slot], k, v, rope), stream);
  if (s != KVC_OK) return s;
  if (r->cfg.source_tokens > 0) {
    // rows n.. of the caller's tensors (and of the rotation table) are the
    // chunk's source tokens
    const size_t n = static_cast<size_t>(r->cfg.chunk_tokens);
    const size_t skip = n * r->cfg.heads * r->cfg.head_dim * 2;
    s = launch_cache_write(write_desc(r, r->L.source, static_cast<const char*>(k) + skip,
                                      static_cast<const char*>(v) + skip,
                                      rope ? rope + n * r->cfg.head_dim : nullptr),
                           stream);
    if (s != KVC_OK) return s;
  }
  r->current = slot;
  if (kind == KVC_STAGE) {
    r->staging = slot;
    r->phase = KVC_PHASE_STAGED;
    return KVC_OK;
  }
  // COMMIT: publish as the sink (chunk 0) or the newest window chunk
  r->slot_chunk[slot] = r->t;
  if (r->t == 0) {
    r->sink_slot = slot;
  } else {
    r->win_id[r->n_win] = r->t;
    r->win_slot[r->n_win] = slot;
    ++r->n_win;
  }
  r->staging = -1;
  r->phase = KVC_PHASE_COMMITTED;
  return KVC_OK;
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" {

size_t kvc_required_bytes(const kvc_config* cfg) {
  if (!config_ok(cfg)) return 0;
  return make_layout(*cfg).total;
}

kvc_status kvc_create(const kvc_config* cfg, void* dev_buf, size_t bytes, kvc_ring** out) {
  if (!out) return KVC_E_INVAL;
  if (!config_ok(cfg) || !dev_buf) return KVC_E_INVAL;
  if (reinterpret_cast<uintptr_t>(dev_buf) % KVC_ALIGN) return KVC_E_INVAL;
  Layout L = make_layout(*cfg);
  if (bytes < L.total) return KVC_E_NOMEM;
  kvc_ring* r = new (std::nothrow) kvc_ring();
  if (!r) return KVC_E_NOMEM;
  r->cfg = *cfg;
  r->L = L;
  r->base = static_cast<unsigned char*>(dev_buf);
  r->scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale
                                      : 1.0f / std::sqrt(static_cast<float>(cfg->head_dim));
  for (int i = 0; i < KVC_MAX_WINDOW + 2; ++i) r->slot_chunk[i] = -1;
  r->sink_slot = -1;
  r->n_win = 0;
  r->t = 0;
  r->phase = KVC_PHASE_EMPTY;
  r->staging = -1;
  r->current = -1;
  r->cond_valid = 0;
  r->ref_valid = 0;
  *out = r;
  return KVC_OK;
}

kvc_status chunk_attn_fwd(kvc_ring* r, const void* q, void* o, float* lse, void* stream) {
  return attention_call(r, q, o, lse, nullptr, nullptr, nullptr, stream);
}

kvc_status chunk_attn_fwd_noalloc(kvc_ring* r, const void* q, void* o, float* lse,
                                  void* stream) {
  return attention_call(r, q, o, lse, nullptr, nullptr, nullptr, stream, true);
}

kvc_status chunk_attn_fwd_rows(kvc_ring* r, const void* q, void* o, float* lse,
                               const int32_t* rows, const int32_t* count, void* stream) {
  if (!rows || !count || !aligned4(rows) || !aligned4(count)) return KVC_E_INVAL;
  return attention_call(r, q, o, lse, nullptr, rows, count, stream);
}

kvc_status chunk_attn_fwd_rope(kvc_ring* r, const void* q, void* o, float* lse,
                               const float* rope, const int32_t* rows, const int32_t* count,
                               void* stream) {
  if ((rows == nullptr) != (count == nullptr)) return KVC_E_INVAL;
  if (rows && (!aligned4(rows) || !aligned4(count))) return KVC_E_INVAL;
  return attention_call(r, q, o, lse, rope, rows, count, stream);
}

kvc_status kvc_append_chunk(kvc_ring* r, int32_t kind, const void* k, const void* v,
                            void* stream) {
  return append(r, kind, k, v, nullptr, stream);
}

kvc_status kvc_append_chunk_rope(kvc_ring* r, int32_t kind, const void* k, const void* v,
                                 const float* rope, void* stream) {
  return append(r, kind, k, v, rope, stream);
}

kvc_status kvc_edit_mask(const void* z_src, const void* z_edit, int32_t tokens, int32_t channels,
                         float tau, int32_t keep, int32_t* rows, int32_t* count, void* stream) {
  if (!z_src || !z_edit || !rows || !count) return KVC_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(z_src) & 1u) || (reinterpret_cast<uintptr_t>(z_edit) & 1u) ||
      !aligned4(rows) || !aligned4(count))
    return KVC_E_INVAL;
  if (tokens < 1 || tokens > KVC_MAX_MASK_TOKENS) return KVC_E_INVAL;
  if (channels < 1 || channels > KVC_MAX_MASK_CHANNELS) return KVC_E_INVAL;
  if (keep < 0 && !(tau >= 0.f)) return KVC_E_INVAL;     // negative or NaN
  EditMaskDesc d;
  d.z_src = z_src;
  d.z_edit = z_edit;
  d.tokens = tokens;
  d.channels = channels;
  d.tau = tau;
  d.keep = keep < 0 ? -1 : keep;
  d.rows = rows;
  d.count = count;
  return launch_edit_mask(d, stream);
}

kvc_status kvc_evict(kvc_ring* r, int32_t* evicted) {
  if (!r) return KVC_E_INVAL;
  if (r->phase == KVC_PHASE_STAGED) return KVC_E_STATE;
  int dropped = -1;
  if (r->phase == KVC_PHASE_COMMITTED) {
    if (r->n_win > r->cfg.window) {
      dropped = r->win_id[0];
      r->slot_chunk[r->win_slot[0]] = -1;
      for (int i = 1; i < r->n_win; ++i) {
        r->win_id[i - 1] = r->win_id[i];
        r->win_slot[i - 1] = r->win_slot[i];
      }
      --r->n_win;
    }
    r->t += 1;
    r->phase = KVC_PHASE_EMPTY;
    r->current = -1;
  }
  if (evicted) *evicted = dropped;
  return KVC_OK;
}

kvc_status kvc_destroy(kvc_ring* r) {
  delete r;
  return KVC_OK;
}

const char* kvc_status_str(kvc_status s) {
  switch (s) {
    case KVC_OK: return "KVC_OK";
    case KVC_E_INVAL: return "KVC_E_INVAL: invalid argument";
    case KVC_E_STATE: return "KVC_E_STATE: call not allowed in the ring's current state";
    case KVC_E_NOMEM: return "KVC_E_NOMEM: buffer smaller than kvc_required_bytes";
    case KVC_E_DEVICE: return "KVC_E_DEVICE: HIP runtime error";
    case KVC_E_UNSUPPORTED: return "KVC_E_UNSUPPORTED: not supported by this library";
    case KVC_E_SCRATCH:
      return "KVC_E_SCRATCH: call needs more than the static scratch of chunk_attn_fwd_noalloc "
             "(KVC_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown kvc status";
  }
}

kvc_status kvc_get_info(const kvc_ring* r, kvc_info* out) {
  if (!r || !out) return KVC_E_INVAL;
  kvc_info i;
  std::memset(&i, 0, sizeof(i));
  i.chunk = r->t;
  i.phase = r->phase;
  i.cond_valid = r->cond_valid;
  i.ref_valid = r->ref_valid;
  i.sink_valid = r->sink_slot >= 0;
  i.n_window = r->n_win;
  kvc_segment segs[kMaxSegments];
  int n = segment_table(r, segs, nullptr);
  if (n > 0) {
    i.n_segments = n;
    for (int s = 0; s < n; ++s) i.kv_len += segs[s].rows;
  }
  for (int s = 0; s < r->L.n_slots; ++s)
    if (r->slot_chunk[s] < 0 && s != r->staging) ++i.free_slots;
  *out = i;
  return KVC_OK;
}

kvc_status kvc_get_segments(const kvc_ring* r, kvc_segment* out, int32_t cap, int32_t* count) {
  if (!r || !count || cap < 0 || (cap > 0 && !out)) return KVC_E_INVAL;
  kvc_segment segs[kMaxSegments];
  int n = segment_table(r, segs, nullptr);
  if (n < 0) return KVC_E_STATE;
  for (int s = 0; s < n && s < cap; ++s) out[s] = segs[s];
  *count = n;
  return KVC_OK;
}

kvc_status kvc_get_slot(const kvc_ring* r, int32_t which, kvc_slot_view* out) {
  if (!r || !out) return KVC_E_INVAL;
  const SlotGeom* g = nullptr;
  if (which == -1) {
    if (r->cfg.cond_tokens <= 0 || !r->cond_valid) return KVC_E_STATE;
    g = &r->L.cond;
  } else if (which == -2) {
    if (r->current < 0) return KVC_E_STATE;
    g = &r->L.chunk[r->current];
  } else if (which == -3) {
    if (r->cfg.ref_tokens <= 0 || !r->ref_valid) return KVC_E_STATE;
    g = &r->L.ref;
  } else if (which == -4) {
    if (r->cfg.source_tokens <= 0 || r->current < 0) return KVC_E_STATE;
    g = &r->L.source;
  } else if (which >= 0) {
    for (int s = 0; s < r->L.n_slots; ++s)
      if (r->slot_chunk[s] == which) g = &r->L.chunk[s];
    if (!g) return KVC_E_STATE;
  } else {
    return KVC_E_INVAL;
  }
  kvc_slot_view v;
  std::memset(&v, 0, sizeof(v));
  v.k = r->base + g->k_off;
  v.vt = r->base + g->vt_off;
  if (r->cfg.kv_dtype == KVC_KV_FP8_E4M3) {
    v.k_scale = reinterpret_cast<float*>(r->base + g->scale_off);
    v.v_scale = v.k_scale + r->cfg.heads;
  }
  v.rows = g->rows;
  v.pitch = g->pitch;
  v.elem_bytes = r->cfg.kv_dtype == KVC_KV_FP8_E4M3 ? 1 : 2;
  *out = v;
  return KVC_OK;
}

}  // extern "C"
