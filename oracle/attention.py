"""O1: chunk-causal sink+window attention as its plain definition (fp64).

Test infrastructure only (see the package docstring).

What is computed, for one layer and one chunk t (discuss.pytorch.kr,
"JoyAI-Video-Edit 소개", chunk-wise autoregressive adaptation section and the
real-time deployment section; ta-paperlens section 4.1):

1. The visible key/value set is assembled explicitly, in logical order:
   condition tokens, then the sink (chunk 0, once t >= 1), then the window of
   the W most recent earlier chunks (oldest first), then chunk t itself.
2. Softmax attention of chunk t's queries over that whole set, per head:
   z_j = scale * <q, k_j>, mu = max_j z_j, p_j = exp(z_j - mu),
   l = sum_j p_j, o = sum_j p_j v_j / l, lse = mu + ln l.

No tiling, no online softmax, no reordering: full score matrix in float64.
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


def kv_length(t: int, cond_tokens: int, chunk_tokens: int, window: int) -> int:
    """Number of keys chunk ``t`` attends: condition + visible chunks + itself."""
    return cond_tokens + chunk_tokens * (len(visible_chunks(t, window)) + 1)


def as_f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or a (CPU) torch tensor."""
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def assemble_kv(cond: np.ndarray | None, history: list[np.ndarray],
                current: np.ndarray) -> np.ndarray:
    """Concatenate [cond ; history... ; current] along the token axis."""
    parts = []
    if cond is not None and cond.shape[0] > 0:
        parts.append(cond)
    parts.extend(history)
    parts.append(current)
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


def chunk_attention(q, cond_k, cond_v, hist_k: list, hist_v: list, cur_k, cur_v,
                    scale: float, return_probs: bool = False):
    """Attention of one chunk's queries over [cond ; history ; current].

    ``hist_k``/``hist_v`` are the clean K/V of the visible earlier chunks in
    logical order (sink first, then window oldest to newest), as returned by
    :func:`visible_chunks`.  ``cond_k``/``cond_v`` may be None (no condition
    tokens).
    """
    K = assemble_kv(None if cond_k is None else as_f64(cond_k),
                    [as_f64(x) for x in hist_k], as_f64(cur_k))
    V = assemble_kv(None if cond_v is None else as_f64(cond_v),
                    [as_f64(x) for x in hist_v], as_f64(cur_v))
    return softmax_attention(q, K, V, scale, return_probs=return_probs)


class StreamOracle:
    """Keeps committed clean K/V per chunk id and answers per-chunk attention.

    Holds every committed chunk (no eviction): which chunks are visible is
    decided by :func:`visible_chunks` alone, independently of any cache.
    """

    def __init__(self, window: int, scale: float, cond_k=None, cond_v=None):
        self.window = window
        self.scale = scale
        self.cond_k = None if cond_k is None else as_f64(cond_k)
        self.cond_v = None if cond_v is None else as_f64(cond_v)
        self.clean: dict[int, tuple[np.ndarray, np.ndarray]] = {}

    def commit(self, t: int, k, v) -> None:
        self.clean[t] = (as_f64(k), as_f64(v))

    def attend(self, t: int, q, cur_k, cur_v, return_probs: bool = False):
        ids = visible_chunks(t, self.window)
        hist_k = [self.clean[j][0] for j in ids]
        hist_v = [self.clean[j][1] for j in ids]
        return chunk_attention(q, self.cond_k, self.cond_v, hist_k, hist_v,
                               cur_k, cur_v, self.scale, return_probs)
