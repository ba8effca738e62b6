"""O1: chunk-causal sink+window attention as its plain definition (fp64).

Test infrastructure only (see the package docstring).

What is computed, for one layer and one chunk t (discuss.pytorch.kr,
"JoyAI-Video-Edit 소개", chunk-wise autoregressive adaptation section and the
real-time deployment section; ta-paperlens section 4.1):

1. The visible key/value set is assembled explicitly, in logical order:
   condition tokens, then the reference tokens (if any), then the sink
   (chunk 0, once t >= 1), then the window of the W most recent earlier
   chunks (oldest first), then chunk t itself, then chunk t's source tokens
   (if any).
2. Softmax attention of chunk t's queries (its own tokens, then its source
   tokens) over that whole set, per head:
   z_j = scale * <q, k_j>, mu = max_j z_j, p_j = exp(z_j - mu),
   l = sum_j p_j, o = sum_j p_j v_j / l, lse = mu + ln l.

No tiling, no online softmax, no reordering: full score matrix in float64.

Token groups (same page, architecture section: the noise, global, history,
condition, reference and source groups and the mask between them; chunk-wise
adaptation section: the active chunk sees its source and condition tokens
bidirectionally, the windowed history and the sink causally, and only the
reference tokens are open to every chunk).  Readings: the reference tokens are
keys/values visible to every chunk, like the condition tokens; the source
tokens of chunk t are queried with chunk t and see exactly what chunk t's own
tokens see (so the two attend each other); earlier chunks' source tokens are
not part of the history.
"""
from __future__ import annotations

import numpy as np


def visible_chunks(t: int, window: int) -> list[int]:
    """Ids of the earlier chunks chunk ``t`` attends, in logical order.

    The first chunk (id 0) is the global sink and stays visible to every later
    chunk; besides it, the ``window`` most recent earlier chunks are visible,
    oldest first.  Chunk 0 is listed once, as the sink (window ids start at 1).
    Chunk ``t`` itself (the current chunk) is not part of this list.
    """
    if t < 0 or window < 0:
        raise ValueError("t and window must be non-negative")
    past = [0] if t >= 1 else []
    past.extend(range(max(1, t - window), t))
    return past


def kv_length(t: int, cond_tokens: int, chunk_tokens: int, window: int,
              ref_tokens: int = 0, source_tokens: int = 0) -> int:
    """Number of keys chunk ``t`` attends: condition + reference + visible
    chunks + itself + its source tokens."""
    return (cond_tokens + ref_tokens + chunk_tokens * (len(visible_chunks(t, window)) + 1)
            + source_tokens)


def as_f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or a (CPU) torch tensor."""
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def assemble_kv(cond: np.ndarray | None, history: list[np.ndarray],
                current: np.ndarray, ref: np.ndarray | None = None,
                source: np.ndarray | None = None) -> np.ndarray:
    """Concatenate [cond ; ref ; history... ; current ; source] along the
    token axis (absent or empty groups are skipped)."""
    parts = []
    for x in (cond, ref):
        if x is not None and x.shape[0] > 0:
            parts.append(x)
    parts.extend(history)
    parts.append(current)
    if source is not None and source.shape[0] > 0:
        parts.append(source)
    return np.concatenate(parts, axis=0)


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                      return_probs: bool = False):
    """Naive softmax attention per head, float64.

    q: [n, H, d]; k, v: [S, H, d].  Returns o [n, H, d] and lse [H, n]
    (natural log), plus the probability matrix [H, n, S] when asked.
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    n, H, d = q.shape
    S = k.shape[0]
    o = np.empty((n, H, d), dtype=np.float64)
    lse = np.empty((H, n), dtype=np.float64)
    probs = np.empty((H, n, S), dtype=np.float64) if return_probs else None
    for h in range(H):
        z = scale * (q[:, h, :] @ k[:, h, :].T)          # [n, S] scores
        mu = z.max(axis=1, keepdims=True)                 # row max
        p = np.exp(z - mu)                                # shifted exponentials
        l = p.sum(axis=1, keepdims=True)                  # row sums
        o[:, h, :] = (p @ v[:, h, :]) / l
        lse[h] = mu[:, 0] + np.log(l[:, 0])
        if return_probs:
            probs[h] = p / l
    if return_probs:
        return o, lse, probs
    return o, lse


def _opt(x):
    return None if x is None else as_f64(x)


def chunk_attention(q, cond_k, cond_v, hist_k: list, hist_v: list, cur_k, cur_v,
                    scale: float, return_probs: bool = False, ref_k=None, ref_v=None,
                    src_k=None, src_v=None):
    """Attention of one chunk's queries over [cond ; ref ; history ; current ;
    source].

    ``hist_k``/``hist_v`` are the clean K/V of the visible earlier chunks in
    logical order (sink first, then window oldest to newest), as returned by
    :func:`visible_chunks`.  ``cond_*``, ``ref_*`` and ``src_*`` may be None
    (no such tokens).  ``q`` holds the chunk's own queries followed by its
    source tokens' queries when there are source tokens.
    """
    K = assemble_kv(_opt(cond_k), [as_f64(x) for x in hist_k], as_f64(cur_k),
                    _opt(ref_k), _opt(src_k))
    V = assemble_kv(_opt(cond_v), [as_f64(x) for x in hist_v], as_f64(cur_v),
                    _opt(ref_v), _opt(src_v))
    return softmax_attention(q, K, V, scale, return_probs=return_probs)


class StreamOracle:
    """Keeps committed clean K/V per chunk id and answers per-chunk attention.

    Holds every committed chunk (no eviction): which chunks are visible is
    decided by :func:`visible_chunks` alone, independently of any cache.
    """

    def __init__(self, window: int, scale: float, cond_k=None, cond_v=None, ref_k=None,
                 ref_v=None):
        self.window = window
        self.scale = scale
        self.cond_k = _opt(cond_k)
        self.cond_v = _opt(cond_v)
        self.ref_k = _opt(ref_k)
        self.ref_v = _opt(ref_v)
        self.clean: dict[int, tuple[np.ndarray, np.ndarray]] = {}

    def commit(self, t: int, k, v) -> None:
        self.clean[t] = (as_f64(k), as_f64(v))

    def attend(self, t: int, q, cur_k, cur_v, return_probs: bool = False, src_k=None,
               src_v=None):
        ids = visible_chunks(t, self.window)
        hist_k = [self.clean[j][0] for j in ids]
        hist_v = [self.clean[j][1] for j in ids]
        return chunk_attention(q, self.cond_k, self.cond_v, hist_k, hist_v,
                               cur_k, cur_v, self.scale, return_probs,
                               self.ref_k, self.ref_v, src_k, src_v)
