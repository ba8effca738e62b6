/*
 * kvc.h -- chunk-causal sink+window attention over a bounded KV cache, gfx950.
 *
 * The method (JoyAI-Video-Edit): a video stream is cut into chunks (one latent
 * frame = 8 video frames each).  The queries of the chunk being generated
 * attend
 *   - every key of their own chunk (bidirectional inside the chunk),
 *   - the condition tokens (always visible),
 *   - the first chunk of the stream, kept as a global sink, and
 *   - a sliding window of the W most recent earlier chunks,
 * so the attended set, and with it per-chunk cost and memory, stays bounded
 * however long the stream runs.  After a chunk is generated its clean K/V is
 * cached for later chunks; the cache keeps only the sink and the window.
 *
 * Two more token groups of the same model are optional: reference tokens R
 * (an optional reference image's latent tokens, visible to every chunk, like
 * the condition tokens) and the source tokens S_t of the chunk being edited
 * (the aligned source-video chunk).  The active chunk sees its own source
 * tokens bidirectionally; they are queried together with the chunk's own
 * tokens and are never cached as history.  Source: discuss.pytorch.kr
 * "JoyAI-Video-Edit 소개", the token-group paragraphs of the architecture
 * section (noise, global, history, condition, reference and source groups
 * and the attention mask between them) and of the chunk-wise adaptation
 * section (visibility of each group from the active chunk).
 * Sources: discuss.pytorch.kr "JoyAI-Video-Edit 소개", sections on the
 * chunk-wise autoregressive adaptation (paper section 4.1) and the real-time
 * deployment pipeline (paper section 5); ta-paperlens "論文解説:
 * JoyAI-Video-Edit", sections 4.1 and 5 (per-chunk loop: denoise with the
 * cache as history, then update the cache keeping window + sink).
 *
 * Conventions for every call:
 *   - Status codes are the KVC_* values below; 0 is success, errors are
 *     negative.  After any error the ring's state is unchanged.
 *   - Device pointers are plain HIP device addresses owned by the caller;
 *     the library never allocates device memory and never frees what it is
 *     given.  Streams are hipStream_t passed as void* (NULL = null stream).
 *   - Work is enqueued asynchronously on the given stream; no call
 *     synchronises the host with the device.  Calls on one ring must be made
 *     from one host thread in program order, and their device work must be
 *     ordered (same stream, or ordered by the caller).  Distinct rings are
 *     independent.
 *   - Tensors are row-major, token-major bf16 unless stated:
 *     [rows][heads][head_dim], contiguous, 16-byte aligned base.
 *   - Inputs holding NaN or Inf are not checked; they propagate.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvc_status;
#define KVC_OK             0
#define KVC_E_INVAL       (-1)  /* bad argument: config, null or misaligned pointer */
#define KVC_E_STATE       (-2)  /* call not allowed in the ring's current state */
#define KVC_E_NOMEM       (-3)  /* caller buffer smaller than kvc_required_bytes */
#define KVC_E_DEVICE      (-4)  /* the HIP runtime reported an error */
#define KVC_E_UNSUPPORTED (-5)  /* valid request this library does not implement */
#define KVC_E_SCRATCH     (-6)  /* chunk_attn_fwd_noalloc: needs more than its static scratch */

/* K/V storage type of a ring */
#define KVC_KV_BF16      0   /* bf16, bit copies of the caller's K/V */
#define KVC_KV_FP8_E4M3  1   /* OCP E4M3 codes + one float32 scale per (head, stored chunk) */

/* kinds for kvc_append_chunk */
#define KVC_COND    0   /* condition tokens (m rows) */
#define KVC_STAGE   1   /* K/V of the current chunk for the present denoise step */
#define KVC_COMMIT  2   /* clean K/V of the current chunk, kept as history */
#define KVC_REF     3   /* reference tokens (r rows), always visible */

/* ring phases reported by kvc_get_info */
#define KVC_PHASE_EMPTY      0   /* no current chunk */
#define KVC_PHASE_STAGED     1   /* current chunk holds staged (noisy) K/V */
#define KVC_PHASE_COMMITTED  2   /* current chunk was committed, not yet evicted */

#define KVC_MAX_WINDOW   29       /* W <= 29 */
#define KVC_MAX_SEGMENTS (KVC_MAX_WINDOW + 5)   /* cond, ref, sink, W window, current, source */
#define KVC_TILE_KEYS    64       /* stored rows are padded to a multiple of this */
#define KVC_MAX_MASK_TOKENS 16384 /* tokens of one kvc_edit_mask call */
#define KVC_MAX_MASK_CHANNELS 4096
#define KVC_ALIGN        256      /* dev_buf alignment */

typedef struct kvc_config {
  int32_t heads;          /* H >= 1 */
  int32_t head_dim;       /* d, 64 or 128 */
  int32_t chunk_tokens;   /* n >= 1: query and key tokens per chunk */
  int32_t cond_tokens;    /* m >= 0: condition tokens (keys/values only) */
  int32_t window;         /* W, 0..KVC_MAX_WINDOW: earlier chunks kept besides the sink */
  int32_t kv_dtype;       /* KVC_KV_BF16 or KVC_KV_FP8_E4M3 */
  float softmax_scale;    /* > 0, or 0 for 1/sqrt(head_dim) */
  int32_t ref_tokens;     /* r >= 0: reference tokens (keys/values only, always visible) */
  int32_t source_tokens;  /* s >= 0: source tokens per chunk (queried and attended with the
                             chunk; never kept as history) */
} kvc_config;

typedef struct kvc_ring kvc_ring;   /* opaque host handle */

/*
 * Bytes of device memory a ring with this config needs (cache slots,
 * per-slot scales, scratch), or 0 if the config is invalid.
 *
 * Layout of dev_buf (for tests and tools; callers only need the size): one
 * slot for the m condition rows (none if m = 0), one for the r reference rows
 * (none if r = 0), W + 2 slots of n rows (sink, W window chunks, one staging
 * slot) and one slot for the s source rows (none if s = 0).  A slot of R rows stores,
 * with P = R rounded up to KVC_TILE_KEYS and e = 2 (bf16) or 1 (fp8) bytes:
 *   K  [H][P][d]  (key-major)        -- rows >= R are zero
 *   Vt [H][P/T][d][T]  (value, transposed in tiles of T keys: T = 32 for
 *                 bf16 rings, 64 for fp8 rings; tile b row j is feature j
 *                 of keys T*b .. T*b+T-1, so one attention step's values are
 *                 one contiguous block) -- columns permuted within tiles:
 *                 bf16 rings: column p holds key kappa(p), where kappa swaps
 *                 bits 2 and 3 of the index (keys permuted within each group
 *                 of 16); fp8 rings: column p (p < 64) of tile b holds key
 *                 64*b + pi(p), pi(p) = ((p & 0x1C) << 1) | ((p & 0x20) >> 3)
 *                 | (p & 3).  Columns of keys >= R are zero.
 *   scales float32 [2][H] (K then V; fp8 rings only)
 * each part starting on a KVC_ALIGN boundary.
 */
size_t kvc_required_bytes(const kvc_config* cfg);

/*
 * Create a ring in caller-owned device memory.
 *   cfg      config as above (copied).
 *   dev_buf  device memory of at least kvc_required_bytes(cfg) bytes, aligned
 *            to KVC_ALIGN.  Owned by the caller; must outlive the ring.  Its
 *            contents need no initialisation.
 *   out      receives the handle.
 * Host-only: no device work, no allocation of device memory.
 * Errors: KVC_E_INVAL (bad config, null pointer, misaligned dev_buf),
 *         KVC_E_NOMEM (bytes < required).
 */
kvc_status kvc_create(const kvc_config* cfg, void* dev_buf, size_t bytes, kvc_ring** out);

/*
 * Write K/V rows into the cache (the fused cache-write kernel).
 *   kind = KVC_COND:   k, v are [m][H][d]; (re)writes the condition slot.
 *                      Allowed in any phase; m must be > 0.
 *   kind = KVC_REF:    k, v are [r][H][d]; (re)writes the reference slot.
 *                      Allowed in any phase; r must be > 0.
 *   kind = KVC_STAGE:  k, v are [n+s][H][d], the current chunk's K/V for this
 *                      denoise step.  From phase EMPTY it takes a free slot
 *                      as staging slot (KVC_E_STATE if none: the previous
 *                      chunk was not evicted); from STAGED it overwrites the
 *                      staging slot (next denoise step).  Not allowed when
 *                      COMMITTED (call kvc_evict first).
 *   kind = KVC_COMMIT: k, v are [n+s][H][d], the clean K/V of the current
 *                      chunk after its denoise steps.  Written into the
 *                      staging slot (or a free slot from phase EMPTY) and
 *                      published: as the sink if this is chunk 0, else as the
 *                      newest window chunk.  Not allowed when already
 *                      COMMITTED.
 *   For STAGE and COMMIT, rows 0..n-1 are the chunk's own tokens and rows
 *   n..n+s-1 its source tokens (s = 0: none), which go to the source slot:
 *   visible to this chunk's attention calls only, never published as history.
 * bf16 rings store bit copies; fp8 rings store E4M3 codes of x/s with
 * s = amax/448 per (head, slot), amax over that head's rows and features,
 * s = 1 when amax = 0 (nearest, ties to even, saturating).
 * The caller's k, v must stay valid until the stream reaches this work.
 * Errors: KVC_E_INVAL (null/misaligned pointers, unknown kind, COND with
 * m = 0, REF with r = 0), KVC_E_STATE, KVC_E_DEVICE.
 */
kvc_status kvc_append_chunk(kvc_ring* ring, int32_t kind, const void* k, const void* v,
                            void* stream);

/*
 * Chunk-causal attention of the current chunk's queries.
 *   q    [n+s][H][d] bf16 queries of the current chunk (its own n tokens,
 *        then its s source tokens).
 *   o    [n+s][H][d] bf16 output, o_i = sum_j softmax_j(scale <q_i, k_j>) v_j
 *        over the visible keys, in logical order [condition ; reference ;
 *        sink (chunk 0, for chunks >= 1) ; window chunks max(1, t-W) .. t-1 ;
 *        current chunk t ; source tokens of chunk t].  Sink and window use
 *        committed clean K/V; the current chunk and its source tokens use the
 *        staged K/V (phase STAGED) or the committed K/V (COMMITTED).
 *   lse  optional [H][n+s] float32 natural-log log-sum-exp of the scaled
 *        logits per query (NULL to skip): that of the weights applied, i.e.
 *        the log of the sum O was normalised by, each weight rounded to the
 *        P type of the product (bf16, or E4M3 for fp8 rings) -- within
 *        ln(1 + 2^-8) of the exact value for bf16 rings.  Merging partial
 *        results by their lse is then exact for the O returned.
 * q may not alias o.  No concatenated KV is formed: the kernel walks the
 * cache slots in logical order.
 * Errors: KVC_E_INVAL (null/misaligned pointers), KVC_E_STATE (phase EMPTY,
 * or condition or reference tokens configured but never written),
 * KVC_E_DEVICE.
 */
kvc_status chunk_attn_fwd(kvc_ring* ring, const void* q, void* o, float* lse, void* stream);

/*
 * chunk_attn_fwd without any device allocation, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, result and errors as chunk_attn_fwd (the
 * same kernels and work split, so the output is bitwise the same); the only
 * difference is where the kernel keeps its split-row scratch (arrival words,
 * partial tags, partial results): in a static device array of the library,
 * KVC_NOALLOC_SCRATCH_BYTES per device, instead of the ring's workspace.
 *   - Each GPU the library runs on holds its own copy of the array until the
 *     process ends; its address is taken once per device (first call with that
 *     device current).  The call allocates and frees nothing.
 *   - Every call on a device shares that device's array, and the array keeps
 *     the last call's contents; only its arrival words and tags must start at
 *     zero, which the first call on the device enqueues (a fill kernel), and
 *     a per-device epoch tells each call's words from older ones.  Calls that
 *     overlap on one device (on concurrent streams, or from several host
 *     threads) race on the array: order them.
 *   - KVC_E_SCRATCH if the call needs more scratch than the array holds
 *     (more than KVC_NOALLOC_MAX_ROWS 128-query rows, i.e. heads *
 *     ceil((n + s) / 128), at head_dim 128).
 */
#define KVC_NOALLOC_MAX_ROWS 8192
#define KVC_NOALLOC_SCRATCH_BYTES (65536u + 4096u + 1048576u + 67108864u)
kvc_status chunk_attn_fwd_noalloc(kvc_ring* ring, const void* q, void* o, float* lse,
                                  void* stream);

/*
 * Rotary position encoding fused into the cache write and the attention's Q
 * load.  Source: discuss.pytorch.kr "JoyAI-Video-Edit 소개", architecture
 * section: every block applies M-RoPE to both streams before the masked
 * self-attention, its angles a fusion of a 3D spatio-temporal RoPE and a 1D
 * source RoPE (no formula given).  The angles are therefore an input:
 *   rope  device float32 [rows][d/2][2], 16-byte aligned: (cos, sin) of the
 *         angle by which features (2i, 2i+1) of each row turn:
 *           x'_{2i} = x_{2i} cos - x_{2i+1} sin,  x'_{2i+1} = x_{2i} sin + x_{2i+1} cos,
 *         each product and the sum/difference a float32 operation rounded on
 *         its own, the result rounded to bf16 (nearest, ties to even), which
 *         is what the kernels then use.  Only keys and queries turn.
 *         NULL: no rotation (the plain calls).
 * kvc_append_chunk_rope: as kvc_append_chunk, with K rotated by rope before
 *   it is stored (rows as the call's k: m, r or n+s; fp8 rings quantise the
 *   rotated keys).
 * chunk_attn_fwd_rope: as chunk_attn_fwd, with q rotated by rope ([n+s] rows)
 *   as it is loaded; rows / count (both NULL, or both given) select active
 *   rows as in chunk_attn_fwd_rows.
 * The result equals the plain calls on K and q rotated beforehand with the
 * arithmetic above.  Errors as for the plain calls; KVC_E_INVAL for a
 * misaligned rope or only one of rows / count.
 */
kvc_status kvc_append_chunk_rope(kvc_ring* ring, int32_t kind, const void* k, const void* v,
                                 const float* rope, void* stream);
kvc_status chunk_attn_fwd_rope(kvc_ring* ring, const void* q, void* o, float* lse,
                               const float* rope, const int32_t* rows, const int32_t* count,
                               void* stream);

/*
 * Attention of selected query rows only (LiveEdit's active rows).
 * Source: aitrends.kr, "LiveEdit 실시간 Diffusion 기반 스트리밍 비디오 편집",
 * AR-oriented Mask Cache (methodology and technical-detail sections): only
 * the tokens whose mask is 1 are recomputed; the others reuse the previous
 * chunk's cached features, here the rows of o left as they are.
 *   q, o, lse  as for chunk_attn_fwd ([n+s][H][d], [H][n+s]); only rows
 *              rows[0 .. *count) of q are read and of o / lse written; every
 *              other row of o and lse keeps its contents.
 *   rows       device int32 [n+s]: row indices, e.g. as written by
 *              kvc_edit_mask.  Indices outside [0, n+s) are skipped; an index
 *              listed twice is computed twice (same result).
 *   count      device int32: number of entries of rows to use, clamped to
 *              [0, n+s].  Read by the kernel, so it may be produced by an
 *              earlier kernel on the stream without a host synchronisation.
 * The result of each selected row is the one chunk_attn_fwd defines (up to
 * rounding: the work split differs).  Errors as for chunk_attn_fwd, and
 * KVC_E_INVAL for null or misaligned rows / count.
 */
kvc_status chunk_attn_fwd_rows(kvc_ring* ring, const void* q, void* o, float* lse,
                               const int32_t* rows, const int32_t* count, void* stream);

/*
 * LiveEdit's active-row mask for the next chunk, on the device.
 * Source: aitrends.kr, "LiveEdit 실시간 Diffusion 기반 스트리밍 비디오 편집",
 * AR-oriented Mask Cache (methodology and technical-detail sections): a
 * token is active where the L2 distance between the previous chunk's edited
 * and source latents exceeds a threshold tau, chosen dynamically so that
 * about 70% of the tokens are pruned.
 *   z_src, z_edit  device bf16 [tokens][channels], token-major.
 *   tokens         1 .. KVC_MAX_MASK_TOKENS;  channels 1 .. KVC_MAX_MASK_CHANNELS.
 *   keep < 0       threshold mode: token i is active iff
 *                    sum_c (z_edit[i][c] - z_src[i][c])^2  >  tau^2,
 *                  the sum taken in float64 over c in increasing order, each
 *                  difference, square and addition rounded on its own, and
 *                  tau^2 = tau * tau in float64 (tau >= 0, not NaN).
 *   keep >= 0      top-k mode (the dynamic threshold): the min(keep, tokens)
 *                  tokens with the largest such sum are active; equal sums
 *                  rank by lower index first.  tau is ignored.
 *                  A NaN sum counts as -1 (never active unless needed to
 *                  reach keep).
 *   rows           device int32 [tokens]: the active token indices in
 *                  increasing order, then -1 up to tokens.
 *   count          device int32 [1]: the number of active tokens.
 * Asynchronous on the stream; no host synchronisation, no allocation.
 * Errors: KVC_E_INVAL (null or misaligned pointers, sizes out of range, bad
 * tau in threshold mode), KVC_E_DEVICE.
 */
kvc_status kvc_edit_mask(const void* z_src, const void* z_edit, int32_t tokens, int32_t channels,
                         float tau, int32_t keep, int32_t* rows, int32_t* count, void* stream);

/*
 * Finish the current committed chunk and recycle cache memory (host only).
 * If more than W window chunks are held, the oldest is dropped and its slot
 * becomes free for the next chunk's staging; the sink is never dropped.
 *   evicted  optional; receives the dropped chunk id, or -1 if none.
 * From phase COMMITTED the ring moves to EMPTY for the next chunk id.  From
 * EMPTY it is a no-op (-1).  From STAGED: KVC_E_STATE.
 */
kvc_status kvc_evict(kvc_ring* ring, int32_t* evicted);

/* Free the host handle (not dev_buf).  NULL is accepted. */
kvc_status kvc_destroy(kvc_ring* ring);

/* Static string naming a status code. */
const char* kvc_status_str(kvc_status status);

/* ---- introspection (host only) ---- */

typedef struct kvc_info {
  int32_t chunk;        /* current chunk id (the next one in phase EMPTY) */
  int32_t phase;        /* KVC_PHASE_* */
  int32_t cond_valid;   /* condition slot written */
  int32_t sink_valid;   /* chunk 0 committed */
  int32_t n_window;     /* committed window chunks held (sink excluded) */
  int32_t kv_len;       /* keys an attention call would attend now, 0 if none */
  int32_t n_segments;   /* segments of that call */
  int32_t free_slots;   /* chunk slots holding nothing */
  int32_t ref_valid;    /* reference slot written */
} kvc_info;

kvc_status kvc_get_info(const kvc_ring* ring, kvc_info* out);

typedef struct kvc_segment {
  int32_t chunk;        /* chunk id (source: the current chunk's), -1 for cond / ref */
  int32_t slot;         /* chunk slot index 0..W+1, -1 cond, -3 ref, -4 source */
  int32_t rows;         /* valid rows */
  int32_t role;         /* 0 cond, 1 sink, 2 window, 3 current, 4 ref, 5 source */
} kvc_segment;

/*
 * The logical segment table an attention call would walk now, in order.
 * Writes at most cap entries to out and the full count to *count.
 * KVC_E_STATE if no attention call is possible now.
 */
kvc_status kvc_get_segments(const kvc_ring* ring, kvc_segment* out, int32_t cap,
                            int32_t* count);

typedef struct kvc_slot_view {
  void* k;              /* K  [H][pitch][d] */
  void* vt;             /* Vt [H][pitch/T][d][T], columns permuted (kappa or pi, see above) */
  float* k_scale;       /* [H] (fp8 rings; NULL for bf16) */
  float* v_scale;       /* [H] */
  int32_t rows;         /* valid rows */
  int32_t pitch;        /* padded rows */
  int32_t elem_bytes;   /* 2 (bf16) or 1 (fp8) */
  int32_t reserved;
} kvc_slot_view;

/*
 * Device addresses of one stored slot, for reading the cache back:
 * which = -1: condition slot; which = -2: the current chunk's slot (staged
 * or committed); which = -3: reference slot; which = -4: source slot (while
 * there is a current chunk); which >= 0: the slot holding that committed
 * chunk id.
 * KVC_E_STATE if that slot holds nothing.
 */
kvc_status kvc_get_slot(const kvc_ring* ring, int32_t which, kvc_slot_view* out);

#ifdef __cplusplus
}
#endif

#endif  /* KVC_H_ */
