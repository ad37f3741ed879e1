"""Comparison helpers for GPU-vs-oracle parity (shared by the GPU tests and smoke()).

Tolerances
  * fp32 path: max |g - r| <= 1e-5 and ||g - r||_2 / ||r||_2 <= 1e-5.
  * bf16 path (bf16 inputs, fp32 accumulation, bf16 output):
      elementwise |g - r| <= 1e-2 + ulp_bf16(r) / 2  and  rel-L2 <= 5e-3,
    where r is the unrounded fp64 oracle. The half-ulp term is the rounding of the
    output itself to bf16 (2^-6 / 2 = 0.0078 for |r| in [2, 4)), which no kernel can
    avoid; the 1e-2 budget is what the kernel's arithmetic may add on top.
"""
from __future__ import annotations

import numpy as np
import torch

BF16_ABS, BF16_REL_L2 = 1e-2, 5e-3
F32_ABS, F32_REL_L2 = 1e-5, 1e-5


def to_f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def ulp_bf16(r: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(r), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def metrics(got, ref) -> dict:
    g, r = to_f64(got), to_f64(ref)
    err = np.abs(g - r)
    denom = max(np.linalg.norm(r), 1e-300)
    return {
        "max_abs": float(err.max()) if err.size else 0.0,
        "rel_l2": float(np.linalg.norm(g - r) / denom) if err.size else 0.0,
        "excess_over_half_ulp": float((err - 0.5 * ulp_bf16(r)).max()) if err.size else 0.0,
        "finite": bool(np.isfinite(g).all()),
    }


def check_bf16(got, ref, what: str = "") -> dict:
    m = metrics(got, ref)
    assert m["finite"], f"{what}: non-finite output"
    assert m["excess_over_half_ulp"] <= BF16_ABS, f"{what}: {m}"
    assert m["rel_l2"] <= BF16_REL_L2, f"{what}: {m}"
    return m


GRAD_REL = 6e-3  # elementwise gradient bar, relative to the tensor's scale


def check_grad(got, ref, what: str = "") -> dict:
    """Gradients of the bf16 backward: rel-L2 <= 5e-3 and |g - r| <= ulp(r)/2 + GRAD_REL max(1,
    max |r|). Every error source of the backward is relative (gradients reach ~40), so the
    elementwise bar is taken relative to the tensor's scale. GRAD_REL = 6e-3 is 1.5x the worst
    error an fp64 emulation of the backward kernels' roundings (backward_rounding_emulation)
    gives on the test inputs (4.1e-3 of the scale over 17 workloads); the emulated roundings
    themselves pass it (tests/test_parity_bars.py)."""
    m = metrics(got, ref)
    assert m["finite"], f"{what}: non-finite output"
    scale = max(1.0, float(np.abs(to_f64(ref)).max())) if to_f64(ref).size else 1.0
    m["excess_over_scale"] = m["excess_over_half_ulp"] / scale
    assert m["excess_over_half_ulp"] <= GRAD_REL * scale, f"{what}: {m}"
    assert m["rel_l2"] <= BF16_REL_L2, f"{what}: {m}"
    return m


def check_f32(got, ref, what: str = "") -> dict:
    m = metrics(got, ref)
    assert m["finite"], f"{what}: non-finite output"
    assert m["max_abs"] <= F32_ABS, f"{what}: {m}"
    assert m["rel_l2"] <= F32_REL_L2, f"{what}: {m}"
    return m


U_BF16 = 2.0 ** -8  # unit roundoff of bf16 (8-bit significand)


def weight_rounding_bound(q, k, v, rho, scale) -> np.ndarray:
    """First-order bound on what rounding the weights to bf16 adds to a causal prefill.

    The kernels round w_j and w_j t_j to bf16 (relative errors e_j, d_j with |e|,|d| <= u)
    and take l and beta from the rounded values. Differentiating
    o = (A1/l)(1 + beta/l) - A2/l gives
        do = sum_j p_j [ e_j ((v_j - vbar)(1 + tbar) + C) + d_j t_j (vbar - v_j) ],
    with C = sum_j p_j (t_j - tbar) v_j, hence
        |do| <= u sum_j p_j ( |v_j - vbar| (|1 + tbar| + |t_j|) + |C| ).
    Returns that bound per output element, [B, H, T, d_v]. It is a worst case (every
    rounding error aligned) and grows with |t|, i.e. with the probe norm; actual errors
    are several times smaller because the individual roundings have random signs.
    """
    q, k, v, rho = (to_f64(x) for x in (q, k, v, rho))
    B, H, T, _ = q.shape
    out = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            a = scale * q[b, h] @ k[b, h].T
            a = np.where(np.tril(np.ones((T, T), bool)), a, -np.inf)
            p = np.exp(a - a.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            t = rho[b, h] @ k[b, h].T
            tbar = (p * t).sum(1)
            vbar = p @ v[b, h]
            C = (p * (t - tbar[:, None])) @ v[b, h]
            dev = np.abs(v[b, h][None, :, :] - vbar[:, None, :])  # [i, j, c]
            fac = np.abs(1 + tbar)[:, None] + np.abs(t)             # [i, j]
            out[b, h] = U_BF16 * (np.einsum("ij,ijc->ic", p * fac, dev) + np.abs(C))
    return out


def sample_rows(B: int, H: int, T: int, n_random: int = 64, seed: int = 0) -> np.ndarray:
    """Flat row ids (b*H + h)*T + i: first rows, tile boundaries, last rows, random rows."""
    rng = np.random.default_rng(seed)
    per_head = set(range(min(8, T)))
    for edge in range(63, T, 64):
        per_head.update({edge, min(edge + 1, T - 1)})
    per_head.update({T - 2, T - 1} if T > 1 else {0})
    per_head = np.array(sorted(i for i in per_head if 0 <= i < T))
    rows = []
    for bh in range(B * H):
        pick = per_head
        if len(pick) > 40:  # keep the explicit-covariance cost bounded on long sequences
            pick = np.concatenate([per_head[:8], per_head[-4:],
                                   rng.choice(per_head, 28, replace=False)])
        rows.append(bh * T + np.unique(np.concatenate([pick, rng.integers(0, T, n_random)])))
    return np.concatenate(rows)


def _bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (through fp32, RNE, as the kernels' conversions)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(
        torch.bfloat16).to(torch.float64).numpy()


def backward_rounding_emulation(q, k, v, rho, scale, do):
    """The causal prefill backward in fp64 with the backward kernels' rounding points, for
    setting the gradient tolerance (not a reference: the reference is oracle.prefill_backward).

    Rounded as in the kernels: the forward's saved vbar and o are bf16, and G_i = <dO_i,
    vbar_i>, D_i = <dO_i, o_i> + tbar_i G_i are formed from them; the pair quantities
    s_ij = p_ij (1 - t_ij + tbar_i), scale * da_ij and dt_ij are rounded to bf16 before the
    products dV = s^T dO, dQ = (scale da) K, dK = (scale da)^T Q + dt^T R, dR = dt K. Everything
    else (p from the saved lse, the sums) is exact here. Returns (dq, dk, dv, drho)."""
    q, k, v, rho, do = (to_f64(a) for a in (q, k, v, rho, do))
    B, H, T, _ = q.shape
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(rho)]
    visible = np.tril(np.ones((T, T), dtype=bool))
    for b in range(B):
        for h in range(H):
            Q, K, V, R, dO = q[b, h], k[b, h], v[b, h], rho[b, h], do[b, h]
            a = np.where(visible, scale * (Q @ K.T), -np.inf)
            p = np.exp(a - a.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            t = np.where(visible, R @ K.T, 0.0)
            tbar = (p * t).sum(axis=1, keepdims=True)
            s = p * (1.0 - t + tbar)
            vbar, o = _bf16(p @ V), _bf16(s @ V)
            g = dO @ V.T
            G = (dO * vbar).sum(axis=1, keepdims=True)
            D = (dO * o).sum(axis=1, keepdims=True) + tbar * G
            sb = _bf16(s)
            dab = _bf16(scale * p * ((1.0 - t + tbar) * g + t * G - D))
            dtb = _bf16(p * (G - g))
            out[2][b, h] = sb.T @ dO
            out[0][b, h] = dab @ K
            out[1][b, h] = dab.T @ Q + dtb.T @ R
            out[3][b, h] = dtb @ K
    return tuple(out)
