"""Rotary position phase (Octopus, Sec. 3.2 Eq. 1).

Eq. 1 says the rotated query-key product depends on the two positions only
through their difference: <R_p q, R_p' k> = Re sum_i z_q,i conj(z_k,i) e^{i (p - p') theta_i}.
The textbook realisation used here pairs dimension i with i + d/2 as the real
and imaginary parts of z_i, with theta_i = base^(-2 i / d) (parity unpinned:
the pages fix neither the pairing nor the base).  Angles and their cosines and
sines are formed in float64.
"""
from __future__ import annotations

import numpy as np


def inv_freq(d: int, base: float) -> np.ndarray:
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def _cos_sin(pos: np.ndarray, d: int, base: float):
    ang = np.asarray(pos, np.float64)[:, None] * inv_freq(d, base)[None, :]
    return np.cos(ang), np.sin(ang)


def rotate(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """R(pos) x for x [T, H, d] (float64 result); base == 0 means no rotation."""
    x = np.asarray(x, np.float64)
    if base == 0:
        return x.copy()
    d = x.shape[-1]
    c, s = _cos_sin(pos, d, base)
    c, s = c[:, None, :], s[:, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rotate_transpose(g: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """R(pos)^T g: the chain rule through the rotation."""
    g = np.asarray(g, np.float64)
    if base == 0:
        return g.copy()
    d = g.shape[-1]
    c, s = _cos_sin(pos, d, base)
    c, s = c[:, None, :], s[:, None, :]
    g1, g2 = g[..., : d // 2], g[..., d // 2:]
    return np.concatenate([g1 * c + g2 * s, g2 * c - g1 * s], axis=-1)
