"""Pins for the fp64 probe producer (oracle.probe) against facts fixed outside it.

* a hand-worked two-head example (tests/golden/probe_two_heads.json), plain and with gamma,
  RoPE and gate [agihunt review, method paragraph: rho = W_R x with its own RMSNorm and
  optional RoPE; mechanism-analysis paragraph: a gate on the probe];
* the RMS of every (token, head) row is sqrt(ms / (ms + eps)) (normalisation per head);
* RoPE keeps each (i, i + d/2) pair's length, leaves a token at position 0 unchanged, and makes the
  dot product of two probes depend only on their position difference;
* W_R = 0 gives rho = 0 (the layer is then plain softmax attention; agihunt review, method
  paragraph).
Each plausible mistake in the producer (normalising over all heads, centring, interleaved
pairs, the opposite rotation, the gate on the wrong axis, the wrong output layout) fails at
least one pin (test_pins_catch_planted_mistakes, which plants them in copies on the CPU).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "probe_two_heads.json"), encoding="utf-8") as fh:
        return json.load(fh)


def _golden_ok(fn) -> bool:
    g = _golden()
    x, w = np.array(g["x"]), np.array(g["w_r"])
    plain = fn(x, w, g["H"], eps=g["eps"])
    full = fn(x, w, g["H"], gamma=g["gamma"], gate=g["gate"], eps=g["eps"],
              rope_base=g["rope_base"])
    return (plain.shape == np.array(g["rho_plain"]).shape
            and np.allclose(plain, g["rho_plain"], rtol=0, atol=g["tol"])
            and np.allclose(full, g["rho_full"], rtol=0, atol=g["tol"]))


def _draw(seed, B=2, T=5, C=12, H=3, d=8):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, T, C)), rng.standard_normal((H * d, C)), H, d


def _rms_ok(fn, seed=0) -> bool:
    x, w, H, d = _draw(seed)
    eps = 1e-3
    rho = fn(x, w, H, eps=eps)                                   # [B, H, T, d]
    y = (x @ w.T).reshape(x.shape[0], x.shape[1], H, d).transpose(0, 2, 1, 3)
    ms = np.mean(y * y, axis=-1)
    return np.allclose(np.sqrt(np.mean(rho * rho, axis=-1)), np.sqrt(ms / (ms + eps)),
                       rtol=1e-12, atol=0)


def _rope_ok(fn, seed=1) -> bool:
    x, w, H, d = _draw(seed)
    base = 500.0
    plain = fn(x, w, H, eps=1e-6)
    rot0 = fn(x, w, H, eps=1e-6, rope_base=base, positions=np.zeros(x.shape[0]))
    rot = fn(x, w, H, eps=1e-6, rope_base=base, positions=np.array([7, 100]))
    half = d // 2
    pair = lambda r: np.hypot(r[..., :half], r[..., half:])  # noqa: E731
    if not np.allclose(rot0[:, :, 0], plain[:, :, 0], rtol=0, atol=1e-14):  # position 0
        return False
    if not np.allclose(pair(rot), pair(plain), rtol=1e-12, atol=1e-14):
        return False
    # Relative positions: the same two tokens at positions (7, 8) and (100, 101) give the
    # same probe dot products (token 0 and token 1 of each sequence, head by head), when the
    # sequences hold the same tokens.
    x2 = np.stack([x[0], x[0]])
    r2 = fn(x2, w, H, eps=1e-6, rope_base=base, positions=np.array([7, 100]))
    dots = np.einsum("bhd,bhd->bh", r2[:, :, 0], r2[:, :, 1])
    return np.allclose(dots[0], dots[1], rtol=1e-10, atol=1e-12)


def _zero_ok(fn) -> bool:
    x, w, H, d = _draw(2)
    return np.array_equal(fn(x, np.zeros_like(w), H, eps=1e-6), np.zeros((2, H, 5, d)))


def _all_pins(fn) -> bool:
    return _golden_ok(fn) and _rms_ok(fn) and _rope_ok(fn) and _zero_ok(fn)


def test_golden_two_heads():
    assert _golden_ok(oracle.probe)


@pytest.mark.parametrize("seed", range(3))
def test_rms_per_head(seed):
    assert _rms_ok(oracle.probe, seed)


@pytest.mark.parametrize("seed", range(3))
def test_rope_rotation_invariants(seed):
    assert _rope_ok(oracle.probe, seed + 1)


def test_zero_projection_gives_zero_probe():
    assert _zero_ok(oracle.probe)


# ------------------------------------------------------------------- planted mistakes
def _mutant(kind):
    def fn(x, w_r, H, gamma=None, gate=None, positions=None, eps=1e-6, rope_base=0.0):
        x = np.asarray(x, float)
        w_r = np.asarray(w_r, float)
        B, T, C = x.shape
        d = w_r.shape[0] // H
        y = (x.reshape(B * T, C) @ w_r.T).reshape(B, T, H, d)
        if kind == "all_heads":
            n = y / np.sqrt(np.mean(y * y, axis=(-2, -1), keepdims=True) + eps)
        elif kind == "centred":
            c = y - y.mean(-1, keepdims=True)
            n = c / np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps)
        else:
            n = y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
        if gamma is not None:
            n = n * np.asarray(gamma, float)
        if rope_base:
            half = d // 2
            i = np.arange(half)
            inv = float(rope_base) ** (-2.0 * i / d)
            p0 = np.zeros(B) if positions is None else np.asarray(positions, float)
            pos = p0[:, None] + np.arange(T)[None, :]
            ang = pos[:, :, None, None] * inv
            sgn = -1.0 if kind == "opposite_turn" else 1.0
            if kind == "interleaved":
                lo, hi = n[..., 0::2], n[..., 1::2]
                out = np.empty_like(n)
                out[..., 0::2] = lo * np.cos(ang) - hi * np.sin(ang)
                out[..., 1::2] = hi * np.cos(ang) + lo * np.sin(ang)
                n = out
            else:
                lo, hi = n[..., :half], n[..., half:]
                n = np.concatenate([lo * np.cos(ang) - sgn * hi * np.sin(ang),
                                    hi * np.cos(ang) + sgn * lo * np.sin(ang)], axis=-1)
        if gate is not None:
            g = np.asarray(gate, float)
            n = n * (g.reshape(1, 1, 1, -1)[..., :d] if kind == "gate_on_dims"
                     else g.reshape(1, 1, H, 1))
        if kind == "token_major":
            return np.ascontiguousarray(n.reshape(B, H, T, d))  # reinterprets [B, T, H, d]
        return np.ascontiguousarray(n.transpose(0, 2, 1, 3))
    return fn


@pytest.mark.parametrize("kind", ["all_heads", "centred", "interleaved", "opposite_turn",
                                  "gate_on_dims", "token_major"])
def test_pins_catch_planted_mistakes(kind):
    assert _all_pins(_mutant("none"))   # the unmutated copy passes, so the harness is sound
    assert not _all_pins(_mutant(kind))
