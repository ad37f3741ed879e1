"""GPU parity of the grouped-query decode (plx_attn_decode_gqa) against the fp64 oracle.

Query head h reads cache head h // G; the oracle runs the plain decode on the cache with
each cache head repeated G times, so it shares nothing with the packed kernel.
"""
import numpy as np
import pytest
import torch

import attention_plx_attn_amd as plx
import oracle
from parity import check_bf16
from plx_synth import decode_inputs
from plx_synth.inputs import DecodeConfig

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, Hq, G, L, seed, rho="scaled", poison=True):
    """q, rho from a decode recipe with H_q heads; the cache from one with H_kv heads (rows at
    or beyond the drawn seqlens poisoned with NaN unless poison=False)."""
    cq = DecodeConfig("dq", 40, B, Hq, 1, 128, "bf16", rho, "full")
    ck = DecodeConfig("dk", 41, B, Hq // G, L, 128, "bf16", rho, "uniform_half")
    xq = decode_inputs(cq, seed=seed)
    xk = decode_inputs(ck, seed=seed, poison=poison)
    return xq["q"], xq["rho"], xk["k_cache"], xk["v_cache"], xk["seqlens"], xq["scale"]


def _oracle(q, rho, kc, vc, sl, scale, G):
    k = torch.nan_to_num(kc.float()).repeat_interleave(G, dim=1)
    v = torch.nan_to_num(vc.float()).repeat_interleave(G, dim=1)
    r = np.zeros(q.shape) if rho is None else rho
    return oracle.decode(q, r, k, v, sl, scale, form="cov")


@pytest.mark.parametrize("probe", ["scaled", "proj32"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("L", [1, 40, 700])
def test_gqa_matches_oracle(G, splits, L, probe):
    B, Hkv = 3, 2
    q, rho, kc, vc, sl, scale = _inputs(B, Hkv * G, G, L, seed=G * 10 + L, rho=probe)
    print("gqa", G, splits, L, probe, sl.tolist(), flush=True)
    o = plx.decode_gqa(q.to(DEV), rho.to(DEV), kc.to(DEV), vc.to(DEV), sl.to(DEV), scale,
                       num_splits=splits)
    torch.cuda.synchronize()
    check_bf16(o, _oracle(q, rho, kc, vc, sl, scale, G),
               f"gqa G={G} splits={splits} L={L} rho={probe}")


@pytest.mark.parametrize("G", [2, 8])
def test_gqa_softmax_only_and_edges(G):
    B, Hkv, L = 5, 2, 200
    q, rho, kc, vc, _, scale = _inputs(B, Hkv * G, G, L, seed=3, poison=False)
    sl = torch.tensor([0, -3, 1, 200, 9999], dtype=torch.int32)
    d = [t.to(DEV) for t in (q, rho, kc, vc, sl)]
    o = plx.decode_gqa(d[0], d[1], d[2], d[3], d[4], scale, num_splits=2)
    z = plx.decode_gqa(d[0], None, d[2], d[3], d[4], scale, num_splits=2)
    z0 = plx.decode_gqa(d[0], torch.zeros_like(d[1]), d[2], d[3], d[4], scale, num_splits=2)
    torch.cuda.synchronize()
    assert torch.equal(z, z0)                       # rho = NULL is rho = 0
    o, z = o.cpu(), z.cpu()
    assert torch.all(o[0] == 0) and torch.all(o[1] == 0)
    for h in range(Hkv * G):                          # one key: exactly its value
        assert torch.equal(o[2, h], vc[2, h // G, 0])
    ref = _oracle(q, rho, kc, vc, sl, scale, G)
    check_bf16(o[3:], ref[3:], f"gqa edges G={G}")
    check_bf16(z[3:], _oracle(q, None, kc, vc, sl, scale, G)[3:], f"gqa softmax-only G={G}")


def test_gqa_g1_equals_plain_decode_oracle_on_32k():
    # G = 1 is the plain multi-head decode; run it on the long-context shape
    from plx_synth import CONFIGS
    cfg = CONFIGS["decode_32k"]
    x = decode_inputs(cfg, seed=0)
    o = plx.decode_gqa(x["q"].to(DEV), x["rho"].to(DEV), x["k_cache"].to(DEV),
                       x["v_cache"].to(DEV), x["seqlens"].to(DEV), x["scale"])
    torch.cuda.synchronize()
    ref = oracle.decode(x["q"], x["rho"], x["k_cache"], x["v_cache"], x["seqlens"], x["scale"],
                        form="sweighted")
    check_bf16(o, ref, "gqa G=1 decode_32k")


def _inputs_d(B, Hq, G, L, d, seed, rho="scaled", poison=True):
    cq = DecodeConfig("dq", 60, B, Hq, 1, d, "bf16", rho, "full")
    ck = DecodeConfig("dk", 61, B, Hq // G, L, d, "bf16", rho, "uniform_half")
    xq = decode_inputs(cq, seed=seed)
    xk = decode_inputs(ck, seed=seed, poison=poison)
    return xq["q"], xq["rho"], xk["k_cache"], xk["v_cache"], xk["seqlens"], xq["scale"]


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("L", [40, 700])
def test_gqa_d64_matches_oracle(G, splits, L):
    """Head dim 64 (the compute-matched head dim) with grouped query heads."""
    B, Hkv = 3, 2
    probe = "proj32" if (G + splits + L) % 2 else "scaled"
    q, rho, kc, vc, sl, scale = _inputs_d(B, Hkv * G, G, L, 64, seed=G * 7 + L, rho=probe)
    print("gqa d64", G, splits, L, probe, sl.tolist(), flush=True)
    o = plx.decode_gqa(q.to(DEV), rho.to(DEV), kc.to(DEV), vc.to(DEV), sl.to(DEV), scale,
                       num_splits=splits)
    torch.cuda.synchronize()
    check_bf16(o, _oracle(q, rho, kc, vc, sl, scale, G),
               f"gqa d64 G={G} splits={splits} L={L} rho={probe}")


@pytest.mark.parametrize("G", [1, 8])
def test_gqa_d64_edges_and_softmax_only(G):
    B, Hkv, L = 5, 2, 200
    q, rho, kc, vc, _, scale = _inputs_d(B, Hkv * G, G, L, 64, seed=5, poison=False)
    sl = torch.tensor([0, -3, 1, 200, 9999], dtype=torch.int32)
    d = [t.to(DEV) for t in (q, rho, kc, vc, sl)]
    o = plx.decode_gqa(d[0], d[1], d[2], d[3], d[4], scale, num_splits=2)
    z = plx.decode_gqa(d[0], None, d[2], d[3], d[4], scale, num_splits=2)
    z0 = plx.decode_gqa(d[0], torch.zeros_like(d[1]), d[2], d[3], d[4], scale, num_splits=2)
    torch.cuda.synchronize()
    assert torch.equal(z, z0)
    o, z = o.cpu(), z.cpu()
    assert torch.all(o[0] == 0) and torch.all(o[1] == 0)
    for h in range(Hkv * G):
        assert torch.equal(o[2, h], vc[2, h // G, 0])
    check_bf16(o[3:], _oracle(q, rho, kc, vc, sl, scale, G)[3:], f"gqa d64 edges G={G}")
    check_bf16(z[3:], _oracle(q, None, kc, vc, sl, scale, G)[3:], f"gqa d64 softmax-only G={G}")


@pytest.mark.parametrize("G", [1, 4, 8])
def test_gqa_one_register_set_instance_matches_two_set_bitwise(G):
    """Sequences of at most 128 rows, one chunk each: a cache of L_max = 128 runs the
    one-register-set instance of the grouped kernel, the same rows in a cache of L_max = 256
    the two-set one; the outputs must be the same bits and within the oracle's bar."""
    B, Hkv, L = 6, 2, 256
    q, rho, kc, vc, _, scale = _inputs(B, Hkv * G, G, L, seed=G + 70, rho="proj32",
                                       poison=False)
    sl = torch.tensor([1, 33, 64, 100, 127, 128], dtype=torch.int32)
    outs = []
    for Lm in (256, 128):
        k = kc[:, :, :Lm].contiguous().to(DEV)
        v = vc[:, :, :Lm].contiguous().to(DEV)
        assert plx.decode_gqa_plan(B, Hkv * G, Hkv, Lm, 128, 1)[0] == 1
        outs.append(plx.decode_gqa(q.to(DEV), rho.to(DEV), k, v, sl.to(DEV), scale,
                                   num_splits=1))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    check_bf16(outs[1], _oracle(q, rho, kc, vc, sl, scale, G), f"gqa one-register-set G={G}")
