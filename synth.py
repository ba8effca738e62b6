"""Seeded synthetic inputs for the chunk-causal attention stream.

This module holds shapes and random draws only: it performs none of the
method's arithmetic (no attention, no softmax, no quantisation).  The oracle
and the HIP path are both fed from here, so they see bit-identical inputs.

Every tensor is drawn from its own numpy stream, keyed by
``SeedSequence([seed, layer, chunk, step, role])``, generated in float32 and
rounded to bfloat16 (round-to-nearest-even, via torch's CPU cast).  The same
(seed, layer, chunk, step, role) therefore always yields the same values,
whatever else the caller generated before; stream-length tests rely on this.

Workloads follow the shapes the JoyAI-Video-Edit pages imply: one chunk is one
latent frame (8 video frames) of a 720x1280 stream, conditioned on MLLM
condition tokens, attended with a global sink plus a sliding window of recent
chunks (discuss.pytorch.kr summary, sections on the chunk-wise autoregressive
adaptation and on real-time deployment).  The head count, head size, tokens per
chunk, condition-token count and window width are not given by the pages; the
values below are the assumed 720p workload (30x54 latent grid = 1620 tokens).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

# role ids for the per-tensor seed streams
ROLES = {
    "q": 0,
    "k_noisy": 1,
    "v_noisy": 2,
    "k_clean": 3,
    "v_clean": 4,
    "k_cond": 5,
    "v_cond": 6,
    "q_src": 7,
    "k_src": 8,
    "v_src": 9,
    "k_src_clean": 10,
    "v_src_clean": 11,
    "k_ref": 12,
    "v_ref": 13,
    "z_src": 14,
    "z_edit": 15,
}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    head_dim: int
    chunk_tokens: int      # n: query tokens per chunk
    cond_tokens: int       # m: condition tokens (KV only, always visible)
    window: int            # W: past chunks kept besides the sink
    chunks: int            # chunks streamed
    steps: int = 1         # denoise steps per chunk (attention calls per layer)
    layers: int = 1        # independent layers, each with its own KV ring
    kv_dtype: str = "bf16"  # "bf16" or "fp8_e4m3"
    std: float = 1.0       # std of the N(0, std^2) draws (baseline distribution)
    seed: int = 0
    ref_tokens: int = 0     # r: reference tokens (KV only, always visible)
    source_tokens: int = 0  # s: source tokens per chunk (queried with the chunk)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS = {
    # 1 head x 64, chunks of 64 tokens, 16 condition tokens, sink + window 2.
    "tiny": Workload("tiny", 1, 64, 64, 16, 2, 6, std=1.0, seed=0),
    # single layer, 720p chunk: 40 heads x 128, 1620 tokens, 256 cond, W=3.
    "720p": Workload("720p", 40, 128, 1620, 256, 3, 16,
                     std=1.0 / math.sqrt(128), seed=1),
    # full depth: 48 layers x 2 denoise steps per chunk, 64 chunks.
    "depth": Workload("depth", 40, 128, 1620, 256, 3, 64, steps=2, layers=48,
                      std=1.0 / math.sqrt(128), seed=2),
    # long stream: W=6, 225 chunks (one minute at 30 fps, 8 frames per chunk).
    "long": Workload("long", 40, 128, 1620, 256, 6, 225,
                     std=1.0 / math.sqrt(128), seed=3),
    # fp8 e4m3 KV cache with per-(head, segment) fp32 scales, Q in bf16.
    "fp8": Workload("fp8", 40, 128, 1620, 256, 3, 32, kv_dtype="fp8_e4m3",
                    std=1.0 / math.sqrt(128), seed=4),
    # all token groups of the editing model at the 720p chunk shape: the
    # chunk's source-video tokens (one latent frame, 1620) are queried and
    # attended with it, and a reference image (one latent frame) is visible to
    # every chunk: 3240 queries over 11596 keys in steady state.
    "groups": Workload("groups", 40, 128, 1620, 256, 3, 16, std=1.0 / math.sqrt(128),
                       seed=5, ref_tokens=1620, source_tokens=1620),
    # chunks of three latent frames (the chunk size of the LiveEdit pages):
    # 4860 tokens per chunk, 256 + 5 * 4860 = 24556 keys in steady state.
    "edit3": Workload("edit3", 40, 128, 4860, 256, 3, 12, std=1.0 / math.sqrt(128),
                      seed=6),
}

# Alternative value distributions for parity runs (std of q, k, v).
# "baseline": the workload's own std for all three.
# "sharp":   N(0,1) for q, k, v   -> logit std ~ 1 at d=128.
# "peaky":   q, k ~ N(0,4), v ~ N(0,1) -> logit std ~ 4 at d=128.
DISTRIBUTIONS = ("baseline", "sharp", "peaky")


def _role_std(w: Workload, dist: str, role: str) -> float:
    if dist == "baseline":
        return w.std
    if dist == "sharp":
        return 1.0
    if dist == "peaky":
        return 1.0 if role.startswith("v") else 2.0
    raise ValueError(f"unknown distribution {dist!r}")


def draw(seed: int, layer: int, chunk: int, step: int, role: str,
         shape: tuple[int, ...], std: float) -> torch.Tensor:
    """One bf16 CPU tensor of N(0, std^2) draws from its own seed stream."""
    ss = np.random.SeedSequence([seed, layer, chunk, step, ROLES[role]])
    rng = np.random.default_rng(ss)
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return torch.from_numpy(x).to(torch.bfloat16)


class Stream:
    """Deterministic per-chunk tensors of one workload.

    Shapes are token-major: q, k, v are [rows, heads, head_dim] bf16.
    ``pool`` > 0 makes chunk and layer indices wrap modulo ``pool`` so that
    long runs can reuse a few pre-uploaded sets (indexed (layer+chunk+step)
    mod pool).
    """

    def __init__(self, w: Workload, dist: str = "baseline", seed: int | None = None,
                 pool: int = 0):
        if dist not in DISTRIBUTIONS:
            raise ValueError(dist)
        self.w = w
        self.dist = dist
        self.seed = w.seed if seed is None else seed
        self.pool = pool
        self._cache: dict = {}

    def _key(self, layer: int, chunk: int, step: int) -> tuple[int, int, int]:
        if self.pool:
            return 0, (layer + chunk + step) % self.pool, 0
        return layer, chunk, step

    def _t(self, layer, chunk, step, role, rows):
        w = self.w
        l, c, s = self._key(layer, chunk, step)
        key = (l, c, s, role)
        if self.pool and key in self._cache:
            return self._cache[key]
        x = draw(self.seed, l, c, s, role, (rows, w.heads, w.head_dim),
                 _role_std(w, self.dist, role))
        if self.pool:
            self._cache[key] = x
        return x

    def q(self, chunk: int, step: int = 0, layer: int = 0) -> torch.Tensor:
        return self._t(layer, chunk, step, "q", self.w.chunk_tokens)

    def kv_noisy(self, chunk: int, step: int = 0, layer: int = 0):
        n = self.w.chunk_tokens
        return (self._t(layer, chunk, step, "k_noisy", n),
                self._t(layer, chunk, step, "v_noisy", n))

    def kv_clean(self, chunk: int, layer: int = 0):
        n = self.w.chunk_tokens
        return (self._t(layer, chunk, 0, "k_clean", n),
                self._t(layer, chunk, 0, "v_clean", n))

    def q_src(self, chunk: int, step: int = 0, layer: int = 0) -> torch.Tensor:
        return self._t(layer, chunk, step, "q_src", self.w.source_tokens)

    def kv_src(self, chunk: int, step: int = 0, layer: int = 0):
        s = self.w.source_tokens
        return (self._t(layer, chunk, step, "k_src", s),
                self._t(layer, chunk, step, "v_src", s))

    def kv_src_clean(self, chunk: int, layer: int = 0):
        s = self.w.source_tokens
        return (self._t(layer, chunk, 0, "k_src_clean", s),
                self._t(layer, chunk, 0, "v_src_clean", s))

    def kv_ref(self, layer: int = 0):
        r = self.w.ref_tokens
        if self.pool:
            layer = layer % self.pool
        return (draw(self.seed, layer, 0, 0, "k_ref", (r, self.w.heads, self.w.head_dim),
                     _role_std(self.w, self.dist, "k_ref")),
                draw(self.seed, layer, 0, 0, "v_ref", (r, self.w.heads, self.w.head_dim),
                     _role_std(self.w, self.dist, "v_ref")))

    def kv_cond(self, layer: int = 0):
        m = self.w.cond_tokens
        if self.pool:
            layer = layer % self.pool
        return (draw(self.seed, layer, 0, 0, "k_cond", (m, self.w.heads, self.w.head_dim),
                     _role_std(self.w, self.dist, "k_cond")),
                draw(self.seed, layer, 0, 0, "v_cond", (m, self.w.heads, self.w.head_dim),
                     _role_std(self.w, self.dist, "v_cond")))


def offset_segment(q: torch.Tensor, k: torch.Tensor, shift: float, scale: float):
    """Input recipe for the segment-offset stress case.

    Sets feature 0 of every query to 1 and feature 0 of every key in ``k`` to
    ``shift / scale``, so that every logit against these keys moves by about
    ``shift`` (exactly by the bf16-rounded amount, which both sides see).
    Returns new tensors; callers apply the zeroing of feature 0 to the other
    segments' keys themselves.
    """
    q = q.clone()
    k = k.clone()
    q[..., 0] = 1.0
    k[..., 0] = shift / scale
    return q, k


def zero_feature0(k: torch.Tensor) -> torch.Tensor:
    k = k.clone()
    k[..., 0] = 0.0
    return k


def edit_latents(seed: int, chunk: int, grid: tuple[int, int], frames: int, channels: int,
                 edit_frac: float = 0.3, background_std: float = 0.05):
    """Synthetic (z_src, z_edit) latents of one chunk for LiveEdit's mask,
    bf16 [frames * rows * cols, channels], token-major (frame, row, col).

    z_src ~ N(0, 1).  z_edit = z_src plus small N(0, background_std^2) noise
    everywhere (the preserved background) and N(0, 1) inside an edited
    rectangle covering about ``edit_frac`` of each frame's grid, placed by the
    seed (the edited object).  Only random draws: no distances, no masking.
    """
    rows, cols = grid
    ss = np.random.SeedSequence([seed, 0, chunk, 0, ROLES["z_src"]])
    rng = np.random.default_rng(ss)
    z_src = rng.standard_normal((frames, rows, cols, channels), dtype=np.float32)
    ss = np.random.SeedSequence([seed, 0, chunk, 0, ROLES["z_edit"]])
    rng = np.random.default_rng(ss)
    noise = rng.standard_normal((frames, rows, cols, channels), dtype=np.float32)
    delta = noise * np.float32(background_std)
    side = math.sqrt(edit_frac)
    h, w = max(1, round(rows * side)), max(1, round(cols * side))
    r0 = int(rng.integers(0, rows - h + 1))
    c0 = int(rng.integers(0, cols - w + 1))
    delta[:, r0:r0 + h, c0:c0 + w, :] = noise[:, r0:r0 + h, c0:c0 + w, :]
    z_edit = z_src + delta
    flat = (frames * rows * cols, channels)
    return (torch.from_numpy(z_src.reshape(flat)).to(torch.bfloat16),
            torch.from_numpy(z_edit.reshape(flat)).to(torch.bfloat16))


def rope_table(seed: int, key: int, rows: int, head_dim: int) -> torch.Tensor:
    """A float32 rotation table [rows, head_dim/2, 2] of (cos, sin) for
    uniformly drawn angles in [-pi, pi): a stand-in for the model's fused
    3D/1D position angles, whose formula the pages do not give."""
    ss = np.random.SeedSequence([seed, key, rows, head_dim, 99])
    ang = np.random.default_rng(ss).uniform(-math.pi, math.pi, (rows, head_dim // 2))
    return torch.from_numpy(np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32))
