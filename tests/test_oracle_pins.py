"""Pins for the fp64 oracle against facts fixed outside the oracle itself.

Every check here runs on the CPU. None of them re-derives the oracle's formula;
each one holds the oracle to a library routine, a closed form worked out by
hand (tests/golden/), or an invariant of the method:

* rho = 0 is exactly softmax attention -> torch's float64 SDPA
  [agihunt review, method paragraph: with W_R = 0 the layer is softmax attention];
* the correction is the softmax-weighted population KV covariance applied to rho
  -> numpy.cov with aweights = scipy softmax weights
  [Resumen Tecnico: Parallax, "Mecanismo Central" equation];
* zero score scale (the infinite-bandwidth limit, agihunt review family paragraph)
  -> plain numpy.cov cross-covariance;
* hand-derived two- and three-key cases (tests/golden/*.json);
* corrected weights sum to one and can be negative or exceed one
  [paper.rainbus.top summary, novelty section];
* a length-1 context returns its only value; translations of k leave o unchanged,
  translations of v shift it; o is affine in rho;
* the three forms (definition, corrected weights, streaming with any block and any
  split merge) agree; decode equals the last causal prefill row and is invariant
  to permuting cache rows; seqlens edge cases.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _draw(seed, B, H, T, dqk, dv, rho_scale=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dqk))
    k = rng.standard_normal((B, H, T, dqk))
    v = rng.standard_normal((B, H, T, dv))
    rho = rng.standard_normal((B, H, T, dqk)) * rho_scale
    return q, k, v, rho


SHAPES = [(1, 2, 17, 4, 4), (2, 1, 33, 16, 16), (1, 1, 64, 16, 8), (1, 2, 40, 8, 12)]


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("shape", SHAPES)
def test_rho_zero_is_softmax_attention(seed, shape):
    B, H, T, dqk, dv = shape
    q, k, v, _ = _draw(seed, B, H, T, dqk, dv)
    rho = np.zeros_like(q)
    scale = 1.0 / np.sqrt(dqk)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True,
        scale=scale).numpy()
    for form in ("cov", "sweighted", "stream"):
        got = oracle.prefill(q, k, v, rho, scale, form=form, block=5)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _weighted_cov_reference(q, k, v, rho, scale):
    """One row: o = vbar - Cov_p(v, k) rho via scipy softmax + numpy.cov(aweights)."""
    p = scipy.special.softmax(scale * (k @ q))
    dv = v.shape[1]
    if k.shape[0] == 1:
        return v[0].copy()
    joint = np.cov(np.hstack([v, k]).T, aweights=p, bias=True)
    cross = joint[:dv, dv:]
    vbar = np.average(v, axis=0, weights=p)
    return vbar - cross @ rho


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("shape", SHAPES)
def test_definition_matches_numpy_weighted_covariance(seed, shape):
    B, H, T, dqk, dv = shape
    q, k, v, rho = _draw(100 + seed, B, H, T, dqk, dv, rho_scale=1.0)
    scale = 1.0 / np.sqrt(dqk)
    got = oracle.prefill(q, k, v, rho, scale, form="cov")
    for b in range(B):
        for h in range(H):
            for i in range(T):
                ref = _weighted_cov_reference(q[b, h, i], k[b, h, : i + 1], v[b, h, : i + 1],
                                              rho[b, h, i], scale)
                np.testing.assert_allclose(got[b, h, i], ref, rtol=0, atol=1e-11)


@pytest.mark.parametrize("seed", range(3))
def test_zero_scale_is_plain_cross_covariance(seed):
    B, H, L, d = 2, 2, 23, 6
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, d))
    rho = rng.standard_normal((B, H, d))
    k = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    seqlens = np.array([L, 11], dtype=np.int32)
    got = oracle.decode(q, rho, k, v, seqlens, 0.0, form="cov")
    for b in range(B):
        n = seqlens[b]
        for h in range(H):
            c = np.cov(v[b, h, :n].T, k[b, h, :n].T, bias=True)[:d, d:]
            ref = v[b, h, :n].mean(0) - c @ rho[b, h]
            np.testing.assert_allclose(got[b, h], ref, rtol=0, atol=1e-12)


def test_golden_two_key():
    g = json.load(open(os.path.join(GOLDEN, "two_key.json")))
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    rho = np.array(g["rho"])[None, None]
    want = np.array(g["o"])
    for form in ("cov", "sweighted", "stream"):
        got = oracle.prefill(q, k, v, rho, g["scale"], form=form, block=1)[0, 0]
        np.testing.assert_allclose(got, want, rtol=0, atol=g["tol"])
    dec = oracle.decode(q[:, :, 1], rho[:, :, 1], k, v, np.array([2], np.int32), g["scale"])
    np.testing.assert_allclose(dec[0, 0], want[1], rtol=0, atol=g["tol"])


def test_golden_three_key_uniform():
    g = json.load(open(os.path.join(GOLDEN, "three_key_uniform.json")))
    q = np.array(g["q"])[None, None]
    rho = np.array(g["rho"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    for form in ("cov", "sweighted", "stream"):
        got = oracle.decode(q, rho, k, v, np.array([3], np.int32), g["scale"], form=form,
                            block=2)
        np.testing.assert_allclose(got[0, 0], g["o"], rtol=0, atol=g["tol"])


@pytest.mark.parametrize("seed", range(3))
def test_corrected_weights_sum_to_one_and_go_negative(seed):
    # With v_j = e_j (one-hot rows, d_v = T) the output row i is the weight row s_i.
    T, d = 24, 8
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 1, T, d))
    k = rng.standard_normal((1, 1, T, d))
    rho = rng.standard_normal((1, 1, T, d)) * 2.0
    v = np.eye(T)[None, None]
    s = oracle.prefill(q, k, v, rho, 1.0 / np.sqrt(d), form="cov")[0, 0]
    np.testing.assert_allclose(s.sum(axis=1), np.ones(T), rtol=0, atol=1e-12)
    assert np.all(np.triu(s, 1) == 0.0), "a future key received weight"
    assert (s < -1e-3).any() and (np.abs(s) > 1.0 + 1e-3).any()
    ones = np.ones((1, 1, T, 5))
    for form in ("cov", "sweighted", "stream"):
        o1 = oracle.prefill(q, k, ones, rho, 0.3, form=form, block=4)
        np.testing.assert_allclose(o1, 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_length_one_context_returns_its_value(seed):
    q, k, v, rho = _draw(200 + seed, 1, 2, 9, 8, 8, rho_scale=3.0)
    for form in ("cov", "sweighted"):
        got = oracle.prefill(q, k, v, rho, 0.7, form=form)
        assert np.array_equal(got[:, :, 0], v[:, :, 0])
        dec = oracle.decode(q[:, :, 3], rho[:, :, 3], k, v, np.array([1], np.int32), 0.7,
                            form=form)
        assert np.array_equal(dec, v[:, :, 0])
    got = oracle.prefill(q, k, v, rho, 0.7, form="stream", block=3)
    np.testing.assert_allclose(got[:, :, 0], v[:, :, 0], rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("seed", range(3))
def test_translation_invariance(seed):
    q, k, v, rho = _draw(300 + seed, 1, 2, 30, 8, 6, rho_scale=1.0)
    rng = np.random.default_rng(seed)
    ck = rng.standard_normal(8) * 3
    cv = rng.standard_normal(6) * 3
    base = oracle.prefill(q, k, v, rho, 0.35, form="cov")
    np.testing.assert_allclose(oracle.prefill(q, k + ck, v, rho, 0.35, form="cov"), base,
                               rtol=0, atol=1e-11)
    np.testing.assert_allclose(oracle.prefill(q, k, v + cv, rho, 0.35, form="cov"), base + cv,
                               rtol=0, atol=1e-11)


@pytest.mark.parametrize("seed", range(3))
def test_affine_in_rho(seed):
    q, k, v, r1 = _draw(400 + seed, 1, 2, 25, 8, 8, rho_scale=1.0)
    r2 = np.random.default_rng(seed).standard_normal(r1.shape)
    f = lambda r: oracle.prefill(q, k, v, r, 0.35, form="cov")  # noqa: E731
    o0, o1, o2, o12 = f(np.zeros_like(r1)), f(r1), f(r2), f(r1 + 2.5 * r2)
    np.testing.assert_allclose(o12 - o0, (o1 - o0) + 2.5 * (o2 - o0), rtol=0, atol=1e-11)
    assert np.abs(o1 - o0).max() > 1e-2  # the correction branch is not silently dropped


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("shape", SHAPES)
def test_forms_agree(seed, shape):
    B, H, T, dqk, dv = shape
    q, k, v, rho = _draw(500 + seed, B, H, T, dqk, dv, rho_scale=1.0)
    scale = 1.0 / np.sqrt(dqk)
    ref = oracle.prefill(q, k, v, rho, scale, form="cov")
    tol = 1e-12 * max(1.0, np.abs(ref).max())
    np.testing.assert_allclose(oracle.prefill(q, k, v, rho, scale, form="sweighted"), ref,
                               rtol=0, atol=tol)
    for block in (1, 3, 7, 16, 64):
        for splits in (1, 2, 3, 7):
            got = oracle.prefill(q, k, v, rho, scale, form="stream", block=block, splits=splits)
            np.testing.assert_allclose(got, ref, rtol=0, atol=tol)


def test_sampled_rows_match_full():
    q, k, v, rho = _draw(7, 2, 3, 21, 8, 8)
    full = oracle.prefill(q, k, v, rho, 0.4, form="sweighted")
    rows = np.array([0, 5, 20, 21, 63, 125])
    got = oracle.prefill(q, k, v, rho, 0.4, form="sweighted", rows=rows)
    np.testing.assert_array_equal(got, full.reshape(-1, 8)[rows])


@pytest.mark.parametrize("seed", range(3))
def test_decode_is_last_prefill_row_and_permutation_invariant(seed):
    B, H, L, d = 3, 2, 37, 8
    q, k, v, rho = _draw(600 + seed, B, H, L, d, d, rho_scale=1.0)
    pre = oracle.prefill(q, k, v, rho, 0.35, form="cov")
    seqlens = np.full(B, L, np.int32)
    dec = oracle.decode(q[:, :, -1], rho[:, :, -1], k, v, seqlens, 0.35, form="cov")
    np.testing.assert_allclose(dec, pre[:, :, -1], rtol=0, atol=1e-12)
    perm = np.random.default_rng(seed).permutation(L)
    decp = oracle.decode(q[:, :, -1], rho[:, :, -1], k[:, :, perm], v[:, :, perm], seqlens,
                         0.35, form="cov")
    np.testing.assert_allclose(decp, dec, rtol=0, atol=1e-12)
    # A shorter seqlens is the prefill row that sees that many keys.
    sl = np.array([1, 17, L], np.int32)
    dec2 = oracle.decode(q[:, :, 16], rho[:, :, 16], k, v, sl, 0.35, form="stream", splits=3)
    np.testing.assert_allclose(dec2[1], pre[1, :, 16], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dec2[0], v[0, :, 0], rtol=1e-14, atol=1e-14)


def test_decode_seqlens_edges():
    B, H, L, d = 4, 2, 10, 4
    q, k, v, rho = _draw(9, B, H, L, d, d)
    qd, rd = q[:, :, 0], rho[:, :, 0]
    sl = np.array([0, -3, 1, 50], np.int32)
    for form in ("cov", "sweighted", "stream"):
        o = oracle.decode(qd, rd, k, v, sl, 0.5, form=form, splits=4)
        assert np.all(o[0] == 0.0) and np.all(o[1] == 0.0)
        np.testing.assert_allclose(o[2], v[2, :, 0], rtol=1e-14, atol=1e-14)
        full = oracle.decode(qd[3:], rd[3:], k[3:], v[3:], np.array([L], np.int32), 0.5,
                             form="cov")
        np.testing.assert_allclose(o[3:], full, rtol=0, atol=1e-12)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_decode_split_merge_matches_definition(splits):
    B, H, L, d = 2, 2, 200, 16
    rng = np.random.default_rng(splits)
    q = rng.standard_normal((B, H, d))
    rho = rng.standard_normal((B, H, d))
    k = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    sl = np.array([200, 61], np.int32)
    ref = oracle.decode(q, rho, k, v, sl, 0.25, form="cov")
    got = oracle.decode(q, rho, k, v, sl, 0.25, form="stream", block=16, splits=splits)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
