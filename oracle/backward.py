"""fp64 backward of the causal Parallax prefill (TEST INFRASTRUCTURE; see the package
docstring for who may use it).

The forward is o_i = sum_j s_ij v_j with s_ij = p_ij (1 - (t_ij - tbar_i)), p = causal
softmax of a_ij = scale <q_i, k_j>, t_ij = <rho_i, k_j>, tbar_i = sum_j p_ij t_ij
[paper.rainbus.top summary, method steps 2-6; agihunt review, method paragraph]. The pages
give no backward formulas; these are the chain rule of that forward, written out per
(b, h) with dense matrices (plain definitions, no blocking):

  g_ij  = <dO_i, v_j>                     G_i = sum_j p_ij g_ij
  dV_j  = sum_i s_ij dO_i
  dt_ij = p_ij (G_i - g_ij)               (t enters s directly and through tbar)
  dp_ij = (1 - t_ij + tbar_i) g_ij + t_ij G_i
  da_ij = p_ij (dp_ij - sum_k p_ik dp_ik) (softmax)
  dQ_i  = scale sum_j da_ij k_j           dK_j = scale sum_i da_ij q_i + sum_i dt_ij rho_i
  dR_i  = sum_j dt_ij k_j

``prefill_stats`` gives the per-row quantities a forward pass saves for the backward
(lse, tbar, vbar).

Pins: tests/test_oracle_backward_pins.py (finite differences of the pinned forward oracle;
torch float64 autograd of softmax attention at rho = 0; dR = -Sigma_KV^T dO, since the
correction is linear in rho; the saved statistics against scipy's logsumexp, the pinned forward
at rho = 0, and that forward with the keys as values).
"""
from __future__ import annotations

import numpy as np


def prefill_stats(q, k, v, rho, scale: float):
    """What a forward pass saves for the backward, per query row of the causal prefill:
    lse_i = ln sum_{j<=i} exp(scale <q_i, k_j>), tbar_i = sum_j p_ij <rho_i, k_j> and
    vbar_i = sum_j p_ij v_j (the softmax-attention output). Returns ([B,H,T], [B,H,T], [B,H,T,d])."""
    q, k, v, rho = (np.asarray(a, dtype=np.float64) for a in (q, k, v, rho))
    B, H, T, _ = q.shape
    lse = np.zeros((B, H, T))
    tbar = np.zeros((B, H, T))
    vbar = np.zeros(v.shape)
    visible = np.tril(np.ones((T, T), dtype=bool))
    for b in range(B):
        for h in range(H):
            a = np.where(visible, scale * (q[b, h] @ k[b, h].T), -np.inf)
            m = a.max(axis=1, keepdims=True)
            e = np.exp(a - m)
            lse[b, h] = (m + np.log(e.sum(axis=1, keepdims=True)))[:, 0]
            p = e / e.sum(axis=1, keepdims=True)
            tbar[b, h] = (p * (rho[b, h] @ k[b, h].T)).sum(axis=1)
            vbar[b, h] = p @ v[b, h]
    return lse, tbar, vbar


def prefill_backward(q, k, v, rho, scale: float, do):
    """Gradients (dq, dk, dv, drho) of sum(do * o) for the causal forward; [B,H,T,d] each."""
    q, k, v, rho, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, rho, do))
    B, H, T, _ = q.shape
    dq, dk, dv, dr = (np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(rho))
    visible = np.tril(np.ones((T, T), dtype=bool))
    for b in range(B):
        for h in range(H):
            Q, K, V, R, dO = q[b, h], k[b, h], v[b, h], rho[b, h], do[b, h]
            a = np.where(visible, scale * (Q @ K.T), -np.inf)
            p = np.exp(a - a.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            t = R @ K.T
            tbar = (p * t).sum(axis=1, keepdims=True)
            s = p * (1.0 - (t - tbar))
            g = dO @ V.T
            G = (p * g).sum(axis=1, keepdims=True)
            dt = p * (G - g)
            dp = (1.0 - t + tbar) * g + t * G
            da = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dv[b, h] = s.T @ dO
            dq[b, h] = scale * (da @ K)
            dk[b, h] = scale * (da.T @ Q) + dt.T @ R
            dr[b, h] = dt @ K
    return dq, dk, dv, dr


__all__ = ["prefill_backward", "prefill_stats"]
