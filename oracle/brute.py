"""O2: whole-stream attention under a block-causal, window-limited mask (fp64).

Test infrastructure only (see the package docstring).  Used to pin O1 on tiny
streams: instead of assembling each chunk's visible keys, the whole stream
[cond | chunk 0 | chunk 1 | ... | chunk T-1] is laid out as one sequence and a
boolean mask decides, for every (query, key) pair, whether the key is visible:

  a query of chunk t may see key j  iff
      j is a condition token, or
      j belongs to chunk 0 (the global sink) or to chunk t itself, or
      j belongs to a chunk c with t - W <= c < t (the sliding window).

This is the mask the JoyAI-Video-Edit pages describe in words
(discuss.pytorch.kr, "JoyAI-Video-Edit 소개", chunk-wise autoregressive
adaptation section: bidirectional within a chunk, causal between chunks,
window of recent chunks plus the first chunk as sink; condition tokens always
visible; future chunks masked).
"""
from __future__ import annotations

import numpy as np


def stream_mask(cond_tokens: int, chunk_tokens: int, chunks: int, window: int) -> np.ndarray:
    """Boolean mask [chunks*chunk_tokens, cond_tokens + chunks*chunk_tokens]."""
    m, n, T = cond_tokens, chunk_tokens, chunks
    q_chunk = np.repeat(np.arange(T), n)                       # chunk of each query
    k_chunk = np.concatenate([np.full(m, -1), np.repeat(np.arange(T), n)])
    qc = q_chunk[:, None]
    kc = k_chunk[None, :]
    is_cond = kc == -1
    is_sink = kc == 0
    is_self = kc == qc
    in_window = (kc >= qc - window) & (kc < qc)
    return is_cond | is_sink | is_self | in_window


def stream_attention(q_chunks: list, k_chunks: list, v_chunks: list,
                     cond_k, cond_v, window: int, scale: float) -> list[np.ndarray]:
    """Per-chunk outputs of masked full-stream attention.

    q_chunks/k_chunks/v_chunks: lists of [n, H, d] arrays, one per chunk (one
    K/V per chunk, so noisy and clean coincide).  cond_k/cond_v: [m, H, d] or
    None.  Returns a list of [n, H, d] float64 outputs.
    """
    T = len(q_chunks)
    n, H, d = np.asarray(q_chunks[0]).shape
    m = 0 if cond_k is None else np.asarray(cond_k).shape[0]
    Q = np.concatenate([np.asarray(x, np.float64) for x in q_chunks], axis=0)
    ks = [np.asarray(x, np.float64) for x in k_chunks]
    vs = [np.asarray(x, np.float64) for x in v_chunks]
    if m:
        ks = [np.asarray(cond_k, np.float64)] + ks
        vs = [np.asarray(cond_v, np.float64)] + vs
    K = np.concatenate(ks, axis=0)
    V = np.concatenate(vs, axis=0)
    mask = stream_mask(m, n, T, window)
    out = np.empty_like(Q)
    for h in range(H):
        z = scale * (Q[:, h, :] @ K[:, h, :].T)
        z = np.where(mask, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        w = np.exp(z)
        w /= w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ V[:, h, :]
    return [out[t * n:(t + 1) * n] for t in range(T)]


# ---- token groups ------------------------------------------------------------
#
# The same whole-stream construction with every token group of the pages'
# attention mask (discuss.pytorch.kr, "JoyAI-Video-Edit 소개", architecture
# section: noise/target, global sink, history, condition, reference and source
# groups; chunk-wise adaptation section: the active chunk sees its source and
# condition tokens bidirectionally, windowed history and the sink causally,
# future chunks are masked, the reference tokens are open to all).
#
# The stream is laid out as
#   [cond | ref | target 0 | source 0 | target 1 | source 1 | ... ]
# and every token carries a (group, chunk) label.  Queries are the target and
# source tokens of every chunk.  A query of chunk t (target or source) may see
#   cond and ref tokens (always),
#   target tokens of chunk 0 (sink), of chunks t-W..t-1 (window) and of t,
#   source tokens of chunk t only.
# Readings: source tokens are queried with their chunk and see what its target
# tokens see; earlier chunks' source tokens are never history.

COND, REF, TARGET, SOURCE = 0, 1, 2, 3


def group_labels(cond_tokens: int, ref_tokens: int, chunk_tokens: int, source_tokens: int,
                 chunks: int) -> tuple[np.ndarray, np.ndarray]:
    """(group, chunk) label of every token of the laid-out stream; chunk is -1
    for cond and ref tokens."""
    groups = [np.full(cond_tokens, COND), np.full(ref_tokens, REF)]
    chunk_ids = [np.full(cond_tokens, -1), np.full(ref_tokens, -1)]
    for t in range(chunks):
        groups += [np.full(chunk_tokens, TARGET), np.full(source_tokens, SOURCE)]
        chunk_ids += [np.full(chunk_tokens, t), np.full(source_tokens, t)]
    return np.concatenate(groups).astype(int), np.concatenate(chunk_ids).astype(int)


def group_mask(key_group: np.ndarray, key_chunk: np.ndarray, query_chunk: np.ndarray,
               window: int) -> np.ndarray:
    """Boolean visibility [queries, keys] from the labels."""
    kg = key_group[None, :]
    kc = key_chunk[None, :]
    qc = query_chunk[:, None]
    always = (kg == COND) | (kg == REF)
    target = (kg == TARGET) & ((kc == 0) | (kc == qc) | ((kc >= qc - window) & (kc < qc)))
    source = (kg == SOURCE) & (kc == qc)
    return always | target | source


def group_stream_attention(q_chunks: list, k_chunks: list, v_chunks: list, cond_k, cond_v,
                           ref_k, ref_v, chunk_tokens: int, window: int,
                           scale: float) -> list[np.ndarray]:
    """Per-chunk outputs of masked whole-stream attention with token groups.

    q_chunks/k_chunks/v_chunks: one [n + s, H, d] array per chunk (the chunk's
    target tokens, then its source tokens; one K/V per chunk, so noisy and
    clean coincide).  cond_*/ref_*: [m, H, d] / [r, H, d] or None.  Returns
    one [n + s, H, d] float64 output per chunk.
    """
    T = len(q_chunks)
    ns, H, d = np.asarray(q_chunks[0]).shape
    n = chunk_tokens
    s = ns - n
    m = 0 if cond_k is None else np.asarray(cond_k).shape[0]
    r = 0 if ref_k is None else np.asarray(ref_k).shape[0]
    kg, kc = group_labels(m, r, n, s, T)
    Q = np.concatenate([np.asarray(x, np.float64) for x in q_chunks], axis=0)
    qc = np.repeat(np.arange(T), ns)
    ks, vs = [], []
    if m:
        ks.append(np.asarray(cond_k, np.float64))
        vs.append(np.asarray(cond_v, np.float64))
    if r:
        ks.append(np.asarray(ref_k, np.float64))
        vs.append(np.asarray(ref_v, np.float64))
    ks += [np.asarray(x, np.float64) for x in k_chunks]
    vs += [np.asarray(x, np.float64) for x in v_chunks]
    K = np.concatenate(ks, axis=0)
    V = np.concatenate(vs, axis=0)
    mask = group_mask(kg, kc, qc, window)
    out = np.empty_like(Q)
    for h in range(H):
        z = scale * (Q[:, h, :] @ K[:, h, :].T)
        z = np.where(mask, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        w = np.exp(z)
        w /= w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ V[:, h, :]
    return [out[t * ns:(t + 1) * ns] for t in range(T)]
