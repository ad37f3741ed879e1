"""Pins for the fp64 backward of the causal prefill (oracle.prefill_backward).

* finite differences: for random directions, the directional derivative of
  L = sum(dO * o) through the pinned forward oracle (central differences in fp64) equals the
  inner product of the gradient with the direction, for q, k, v and rho;
* rho = 0: dq, dk, dv equal torch's float64 autograd through causal scaled-dot-product
  attention (the layer is then softmax attention; agihunt review, method paragraph);
* dR_i = -(Sigma_KV^(i))^T dO_i: the correction is Sigma_KV rho with Sigma_KV independent of
  rho [gist.science summary (Spanish), central equation], checked with numpy.cov weights;
* planted mistakes in copies (a sign, the tbar path, the softmax term) fail the pins;
* the saved statistics (oracle.prefill_stats): lse against scipy.special.logsumexp of the
  visible scores, vbar against the pinned forward at rho = 0 (softmax attention), and tbar as
  <rho_i, kbar_i> with kbar the same forward run with the keys as values.
"""
import scipy.special
import numpy as np
import pytest
import torch

import oracle


def _draw(seed, B=1, H=2, T=9, d=4, rho_scale=0.7):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    rho = rng.standard_normal((B, H, T, d)) * rho_scale
    do = rng.standard_normal((B, H, T, d))
    return q, k, v, rho, do


def _fd_ok(bwd, seed, eps=1e-5, tol=1e-7) -> bool:
    q, k, v, rho, do = _draw(seed)
    scale = 0.6
    grads = bwd(q, k, v, rho, scale, do)
    rng = np.random.default_rng(seed + 100)
    base = [q, k, v, rho]
    for which in range(4):
        delta = rng.standard_normal(base[which].shape)
        plus = [x.copy() for x in base]
        minus = [x.copy() for x in base]
        plus[which] += eps * delta
        minus[which] -= eps * delta
        lp = np.sum(do * oracle.prefill(*plus, scale, form="cov"))
        lm = np.sum(do * oracle.prefill(*minus, scale, form="cov"))
        fd = (lp - lm) / (2 * eps)
        an = np.sum(grads[which] * delta)
        if abs(fd - an) > tol * max(1.0, abs(an)):
            return False
    return True


@pytest.mark.parametrize("seed", range(4))
def test_finite_differences(seed):
    assert _fd_ok(oracle.prefill_backward, seed)


@pytest.mark.parametrize("seed", range(3))
def test_rho_zero_matches_torch_sdpa_autograd(seed):
    q, k, v, _, do = _draw(seed, B=2, H=2, T=13, d=8)
    scale = 0.4
    dq, dk, dv, _ = oracle.prefill_backward(q, k, v, np.zeros_like(q), scale, do)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                         scale=scale)
    o.backward(torch.tensor(do))
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_drho_is_minus_covariance_transpose_times_do(seed):
    q, k, v, rho, do = _draw(seed, T=11, d=5)
    scale = 0.5
    _, _, _, dr = oracle.prefill_backward(q, k, v, rho, scale, do)
    for h in range(q.shape[1]):
        for i in range(q.shape[2]):
            a = scale * (k[0, h, : i + 1] @ q[0, h, i])
            w = np.exp(a - a.max())
            w /= w.sum()
            d = k.shape[-1]
            cov = np.cov(np.concatenate([v[0, h, : i + 1], k[0, h, : i + 1]], axis=1).T,
                         aweights=w, bias=True)[:d, d:] if i > 0 else np.zeros((d, d))
            assert np.allclose(dr[0, h, i], -cov.T @ do[0, h, i], rtol=1e-10, atol=1e-12)


def _mutant(kind):
    def bwd(q, k, v, rho, scale, do):
        B, H, T, _ = q.shape
        out = [np.zeros_like(q) for _ in range(4)]
        vis = np.tril(np.ones((T, T), dtype=bool))
        for h in range(H):
            Q, K, V, R, dO = q[0, h], k[0, h], v[0, h], rho[0, h], do[0, h]
            a = np.where(vis, scale * Q @ K.T, -np.inf)
            p = np.exp(a - a.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            t = R @ K.T
            tbar = (p * t).sum(1, keepdims=True)
            s = p * (1 - (t - tbar))
            g = dO @ V.T
            G = (p * g).sum(1, keepdims=True)
            dt = p * (G - g) if kind != "no_tbar_path" else -p * g
            dp = (1 - t + tbar) * g + t * G
            if kind == "sign_dp":
                dp = (1 + t - tbar) * g + t * G
            da = p * (dp - (p * dp).sum(1, keepdims=True)) if kind != "no_softmax_term" \
                else p * dp
            out[2][0, h] = s.T @ dO
            out[0][0, h] = scale * da @ K
            out[1][0, h] = scale * da.T @ Q + dt.T @ R
            out[3][0, h] = dt @ K
        return tuple(out)
    return bwd


@pytest.mark.parametrize("kind", ["no_tbar_path", "sign_dp", "no_softmax_term"])
def test_pins_catch_planted_mistakes(kind):
    assert _fd_ok(_mutant("none"), 0)
    assert not _fd_ok(_mutant(kind), 0)


@pytest.mark.parametrize("seed", range(3))
def test_saved_statistics(seed):
    q, k, v, rho, _ = _draw(seed, B=2, H=2, T=10, d=6)
    scale = 0.8
    lse, tbar, vbar = oracle.prefill_stats(q, k, v, rho, scale)
    for b in range(2):
        for h in range(2):
            for i in range(10):
                s = scale * (k[b, h, : i + 1] @ q[b, h, i])
                assert np.isclose(lse[b, h, i], scipy.special.logsumexp(s), rtol=1e-13)
    zero = np.zeros_like(rho)
    assert np.allclose(vbar, oracle.prefill(q, k, v, zero, scale, form="cov"), rtol=1e-12,
                       atol=1e-13)
    kbar = oracle.prefill(q, k, k, zero, scale, form="cov")
    assert np.allclose(tbar, np.einsum("bhtd,bhtd->bht", rho, kbar), rtol=1e-12, atol=1e-13)
