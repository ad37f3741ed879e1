"""fp64 probe producer (TEST INFRASTRUCTURE; see the package docstring for who may use it).

rho = gate_h * RoPE(gamma (.) RMSNorm_head(x W_R^T)) in the [B, H, T, d] layout
[agihunt review, method paragraph: rho is one learned projection W_R x of the layer input,
with its own RMSNorm and, optionally, RoPE; gist.science summary (Spanish), method section:
rho_i = W_R x_i; the same review's mechanism-analysis paragraph: a learned gate on the probe].

Each step is written out as its plain definition in float64:
  y      = x W_R^T                                 (a matrix product)
  n      = gamma * y / sqrt(mean_d(y^2) + eps)     (RMSNorm over the d dims of one head)
  RoPE   : dims (i, i + d/2), i < d/2, turned by angle pos * base^(-2 i / d) (rotate-half)
  rho    = gate_h * n
Pins: tests/test_oracle_pins.py (hand-worked example in tests/golden/, invariants).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def probe(x, w_r, H: int, gamma=None, gate=None, positions=None, eps: float = 1e-6,
          rope_base: float = 0.0) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    w_r = np.asarray(w_r, dtype=np.float64)
    B, T, C = x.shape
    HD = w_r.shape[0]
    assert w_r.shape == (HD, C) and HD % H == 0
    d = HD // H
    y = (x.reshape(B * T, C) @ w_r.T).reshape(B, T, H, d)
    n = y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    if gamma is not None:
        n = n * np.asarray(gamma, dtype=np.float64).reshape(1, 1, 1, d)
    if rope_base:
        half = d // 2
        i = np.arange(half, dtype=np.float64)
        inv_freq = float(rope_base) ** (-2.0 * i / d)
        p0 = (np.zeros(B) if positions is None
              else np.asarray(positions, dtype=np.float64).reshape(B))
        pos = p0[:, None] + np.arange(T, dtype=np.float64)[None, :]          # [B, T]
        ang = pos[:, :, None, None] * inv_freq[None, None, None, :]          # [B, T, 1, half]
        lo, hi = n[..., :half], n[..., half:]
        n = np.concatenate([lo * np.cos(ang) - hi * np.sin(ang),
                            hi * np.cos(ang) + lo * np.sin(ang)], axis=-1)
    if gate is not None:
        n = n * np.asarray(gate, dtype=np.float64).reshape(1, 1, H, 1)
    return np.ascontiguousarray(n.transpose(0, 2, 1, 3))                      # [B, H, T, d]


__all__ = ["probe"]
