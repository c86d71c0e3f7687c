"""Oracle: rotary position embedding by tree position ids.  TEST
INFRASTRUCTURE ONLY (see the package docstring).

[TT] section 打包数据的生成: a token's position id is the number of tokens it
may attend to, minus one, which keeps the positional encoding of a shared
prefix the same in every sequence through it; the position ids feed the
model's rotary embedding.  The pages do not spell the rotation out.  This is
the rotation of the Qwen/Llama family the pages train (Qwen3-8B):
for a head vector x of even size D and position p, with
  f_j = base^(-2 j / D),  a_j = p f_j,  j = 0 .. D/2 - 1,
  y_j         = x_j cos a_j - x_{j+D/2} sin a_j,
  y_{j+D/2}   = x_{j+D/2} cos a_j + x_j sin a_j,
and its inverse (sin -> -sin), which is also its gradient map: the rotation
is orthogonal, so the gradient with respect to x is the inverse rotation of
the gradient with respect to y.  Computed in float64.
"""

from __future__ import annotations

import numpy as np


def rope(x: np.ndarray, pos: np.ndarray, base: float, inverse: bool = False) -> np.ndarray:
    """x [L, H, D] (any float dtype), pos [L] -> float64 [L, H, D]."""
    x = np.asarray(x, dtype=np.float64)
    L, H, D = x.shape
    half = D // 2
    j = np.arange(half, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * base ** (-2.0 * j / D)[None, :]  # [L, D/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    if inverse:
        s = -s
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
