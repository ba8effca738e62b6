"""Oracle for chunk-causal sink+window attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation (numpy, float64) of what the
HIP path computes.  It shares no code with the HIP library and imports nothing
from it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it; the product path never does.

Sources (the text of these web pages; the pages print no attention formula or
numeric example, so every function here is the textbook definition of what the
pages describe in words):

* discuss.pytorch.kr, "JoyAI-Video-Edit 소개", section on the chunk-wise
  autoregressive adaptation (paper section 4.1): attention is bidirectional
  inside a chunk and causal across chunks; inter-chunk attention is limited to
  a sliding window of recent chunks plus the first chunk, kept as a global
  sink.  The token-group paragraph of the same section: the active chunk sees
  its condition tokens bidirectionally, clean history and the sink causally,
  future chunks are masked.
* same page, section on the real-time deployment pipeline (paper section 5):
  the clean KV state of a chunk is cached after it is generated; the cache
  keeps the first chunk as sink plus a sliding window, so memory and per-chunk
  compute are bounded for an open-ended stream.
* ta-paperlens, "論文解説: JoyAI-Video-Edit", sections 4.1 and 5 (the per-chunk
  loop: denoise with the cache as history, then update the cache keeping only
  the window and the head sink).
* aitrends.kr, LiveEdit summary, glossary entry on chunk-wise causal attention:
  a chunk sees itself and earlier chunks only; methodology and technical
  detail sections: the AR-oriented Mask Cache (active rows by the L2
  distance of the previous chunk's edited and source latents).

Modules:
  attention  -- O1: explicit KV assembly + fp64 naive softmax attention.
  brute      -- O2: whole-stream attention under a block-causal window mask.
  fp8        -- O3: OCP e4m3 codec and the per-(head, segment) scale rule.
  liveedit   -- O4: LiveEdit's active-row mask and active-row attention.
  rope       -- O5: rotary encoding of Q and K from a per-token angle table.

Readings where the pages are silent (each is listed in the design notes):
  * W counts past chunks only; the sink and the current chunk come on top.
  * chunk 0 appears once, as the sink; window chunks are drawn from 1..t-1.
  * history and sink use committed clean K/V, the current chunk the K/V passed
    for the present denoise step.
  * condition tokens are keys/values only and visible to every chunk.
  * softmax scale is 1/sqrt(head_dim).
  * no masking inside the visible set.

Parity status: every function is pinned by tests in tests/test_oracle.py and
tests/test_fp8_codec.py (brute force, closed forms, library routines,
invariants).  None is "parity unpinned".
"""

from . import attention, brute, fp8, liveedit, rope  # noqa: F401
