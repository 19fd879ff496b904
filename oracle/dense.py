"""Second CPU oracle: dense masked attention in numpy float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

It builds the whole [N, N] score matrix and applies the boolean band mask exactly as the
Sliding Window Attention glossary's example builds it (outer difference of positions,
kept where 0 <= offset < window), widened by the sink columns j < s (Sliding Window
Attention glossary, "attention sink"; Sliding-window beats linear attention, SWA(w, s)).
Scores, bias and weights follow the SWAT page's "Balanced ALiBi" equation; the rotation is
the RoFormer one the SWAT page cites, written with numpy array operations instead of the
C loop's pairwise scalar code.
"""
from __future__ import annotations

import numpy as np

SIGMOID = 0
SOFTMAX = 1


def band_mask(N: int, w: int, s: int = 0) -> np.ndarray:
    """Boolean [N, N] mask: query i (row) may use key j (column)."""
    pos = np.arange(N)
    offset = pos[:, None] - pos[None, :]
    mask = (offset >= 0) & (offset < w)
    if s > 0:
        mask |= (offset >= 0) & (pos[None, :] < s)
    return mask


def rope_dense(x: np.ndarray, theta: float) -> np.ndarray:
    """Rotate x [..., N, H, d] at positions 0..N-1 along axis -3, interleaved pairs."""
    N, d = x.shape[-3], x.shape[-1]
    t = np.arange(d // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * t / d)                       # [d/2]
    ang = np.arange(N, dtype=np.float64)[:, None] * inv_freq  # [N, d/2]
    c = np.cos(ang)[:, None, :]                              # [N, 1, d/2]
    s_ = np.sin(ang)[:, None, :]
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s_
    out[..., 1::2] = xe * s_ + xo * c
    return out


def prefill_dense(q, k, v, *, w: int, s: int = 0, mode: int = SIGMOID, scale: float = 0.0,
                  slopes=None, rope_theta: float = 0.0) -> np.ndarray:
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    if scale <= 0.0:
        scale = 1.0 / np.sqrt(d)
    if rope_theta > 0.0:
        q = rope_dense(q, rope_theta)
        k = rope_dense(k, rope_theta)
    # expand kv heads to query heads: query head h uses kv head h // g
    k = np.repeat(k, g, axis=2)
    v = np.repeat(v, g, axis=2)
    mask = band_mask(N, w, s)
    pos = np.arange(N)
    dist = (pos[:, None] - pos[None, :]).astype(np.float64)   # i - j
    out = np.empty((B, N, Hq, d))
    for h in range(Hq):
        x = np.einsum("bid,bjd->bij", q[:, :, h, :], k[:, :, h, :]) * scale
        if slopes is not None:
            x = x + float(slopes[h]) * dist[None]
        if mode == SIGMOID:
            with np.errstate(over="ignore"):
                p = 1.0 / (1.0 + np.exp(-x))
            p = np.where(mask[None], p, 0.0)
        else:
            xm = np.where(mask[None], x, -np.inf)
            m = xm.max(axis=-1, keepdims=True)
            e = np.exp(xm - m)
            p = e / e.sum(axis=-1, keepdims=True)
        out[:, :, h, :] = np.einsum("bij,bjd->bid", p, v[:, :, h, :])
    return out
