"""O5: rotary position encoding applied to Q and K (test infrastructure only;
see the package docstring).

Source: discuss.pytorch.kr, "JoyAI-Video-Edit 소개", architecture section:
each block applies M-RoPE to both streams before the masked self-attention,
with rotation angles built by fusing a 3D spatio-temporal RoPE and a 1D
source RoPE, so that source and generated tokens take different roles in
one sequence.  The pages give no formula for the angles, so the path takes
the angles as an input: one (cos, sin) pair per token and feature pair, in
a float32 table [rows][d/2][2].  Whatever the model's 3D/1D fusion is, it
only changes that table.

Readings (each listed in the design notes):
  * features (2i, 2i+1) form pair i and turn by the table's angle:
      x'_{2i}   = x_{2i} cos - x_{2i+1} sin
      x'_{2i+1} = x_{2i} sin + x_{2i+1} cos
  * only Q and K turn; V does not;
  * the turned Q and K are held in bf16, the type the kernels consume: each
    product and the sum or difference are float32 operations rounded on their
    own, then the result is rounded to bf16 (nearest, ties to even).  This is
    an encoding, so the oracle takes it in the kernels' precision and the
    stored K is compared bit for bit; the attention itself stays float64 on
    those bf16 values.
"""
from __future__ import annotations

import numpy as np
import torch

from .attention import as_f64


def rotate(x, table) -> np.ndarray:
    """Exact rotation in float64: x [rows, H, d], table [rows, d/2, 2]."""
    x = as_f64(x)
    t = np.asarray(table, dtype=np.float64)
    c = t[:, None, :, 0]
    s = t[:, None, :, 1]
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def rotate_stored(x, table) -> torch.Tensor:
    """The bf16 values the kernels hold for rotated x (bf16 [rows, H, d]):
    float32 products and sum/difference, each rounded, then bf16 RNE."""
    xf = np.asarray(torch.as_tensor(x).to(torch.float32).numpy(), dtype=np.float32)
    t = np.asarray(table, dtype=np.float32)
    c = t[:, None, :, 0]
    s = t[:, None, :, 1]
    xe, xo = xf[..., 0::2], xf[..., 1::2]
    out = np.empty_like(xf)
    a = xe * c
    b = xo * s
    out[..., 0::2] = a - b
    a = xe * s
    b = xo * c
    out[..., 1::2] = a + b
    return torch.from_numpy(out).to(torch.bfloat16)


def table_1d(positions, head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """A plain 1D RoPE table (used by the pins): pair i of a token at
    position p turns by p * theta^(-2i/d)."""
    p = np.asarray(positions, dtype=np.float64)[:, None]
    i = np.arange(head_dim // 2, dtype=np.float64)[None, :]
    ang = p * theta ** (-2.0 * i / head_dim)
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1)
