"""GPU parity of the paged decode with grouped query heads (plx_attn_decode_paged_gqa).

A contiguous cache of H_kv heads is scattered into a block pool in a random order; with the
same split plan the paged call must give the bits of plx_attn_decode_gqa on the contiguous
cache (the arithmetic is the same, only the addresses differ), and match the fp64 oracle run
on the cache with each head repeated G times (query head h reads cache head h // G).
"""
import numpy as np
import pytest
import torch

import attention_plx_attn_amd as plx
import oracle
from paged_cache import paginate
from parity import check_bf16
from plx_synth import decode_inputs
from plx_synth.inputs import DecodeConfig

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, Hkv, G, L, seed, rho="scaled", lengths="uniform_half", poison=True):
    cq = DecodeConfig("pq", 50, B, Hkv * G, 1, 128, "bf16", rho, "full")
    ck = DecodeConfig("pk", 51, B, Hkv, L, 128, "bf16", rho, lengths)
    xq = decode_inputs(cq, seed=seed)
    xk = decode_inputs(ck, seed=seed, poison=poison)
    return xq["q"], xq["rho"], xk["k_cache"], xk["v_cache"], xk["seqlens"], xq["scale"]


def _oracle(q, rho, kc, vc, sl, scale, G):
    k = torch.nan_to_num(kc.float()).repeat_interleave(G, dim=1)
    v = torch.nan_to_num(vc.float()).repeat_interleave(G, dim=1)
    r = np.zeros(q.shape) if rho is None else rho
    return oracle.decode(q, r, k, v, sl, scale, form="cov")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("bs", [32, 64, 256])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_paged_gqa_equals_contiguous_and_oracle(G, bs, splits):
    B, Hkv, L = 3, 2, 1024
    probe = "proj32" if (G + bs // 32 + splits) % 2 else "scaled"
    q, rho, kc, vc, sl, scale = _inputs(B, Hkv, G, L, seed=G * 100 + bs + splits, rho=probe)
    kp, vp, table = paginate(kc, vc, sl, bs, seed=bs + G)
    print("paged gqa", G, bs, splits, probe, sl.tolist(), flush=True)
    d = [t.to(DEV) for t in (q, rho, kp, vp, table, sl)]
    o = plx.decode_paged_gqa(*d, scale, num_splits=splits)
    s = plx.decode_gqa_plan(B, Hkv * G, Hkv, L, 128, splits)[0]
    ref_c = plx.decode_gqa(d[0], d[1], kc.to(DEV), vc.to(DEV), d[5], scale, num_splits=s)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_c)
    check_bf16(o, _oracle(q, rho, kc, vc, sl, scale, G),
               f"paged gqa G={G} bs={bs} splits={splits} rho={probe}")


@pytest.mark.parametrize("G", [2, 8])
def test_paged_gqa_seqlens_edges_and_softmax_only(G):
    B, Hkv, L = 5, 2, 256
    q, rho, kc, vc, _, scale = _inputs(B, Hkv, G, L, seed=7, lengths="full", poison=False)
    sl = torch.tensor([0, -2, 1, 256, 999], dtype=torch.int32)
    kp, vp, table = paginate(kc, vc, sl, 64, seed=G)
    d = [t.to(DEV) for t in (q, rho, kp, vp, table, sl)]
    o = plx.decode_paged_gqa(*d, scale, num_splits=2)
    z = plx.decode_paged_gqa(d[0], None, *d[2:], scale, num_splits=2)
    z0 = plx.decode_paged_gqa(d[0], torch.zeros_like(d[1]), *d[2:], scale, num_splits=2)
    torch.cuda.synchronize()
    assert torch.equal(z, z0)                        # rho = NULL is rho = 0
    o, z = o.cpu(), z.cpu()
    assert torch.all(o[0] == 0) and torch.all(o[1] == 0)
    for h in range(Hkv * G):                          # one key: exactly its value
        assert torch.equal(o[2, h], vc[2, h // G, 0])
    check_bf16(o[3:], _oracle(q, rho, kc, vc, sl, scale, G)[3:], f"paged gqa edges G={G}")
    check_bf16(z[3:], _oracle(q, None, kc, vc, sl, scale, G)[3:],
               f"paged gqa softmax-only G={G}")


@pytest.mark.parametrize("splits", [1, 3, 4, 8])  # 4, 8: one step per wave
def test_paged_gqa_invalid_entry_below_seqlens_is_skipped(splits):
    """An entry outside [0, num_blocks) inside a sequence's valid range: those rows get no
    weight, so the output is the oracle's over the sequence without them."""
    B, Hkv, G, L, bs = 3, 2, 4, 512, 64
    q, rho, kc, vc, sl, scale = _inputs(B, Hkv, G, L, seed=9, rho="proj32", lengths="full")
    kp, vp, table = paginate(kc, vc, sl, bs, seed=11)
    bad = {0: (1, -1), 1: (3, 1 << 30), 2: (0, kp.shape[0])}  # b: (block index, entry)
    for b, (i, entry) in bad.items():
        table[b, i] = entry
    d = [t.to(DEV) for t in (q, rho, kp, vp, table, sl)]
    o = plx.decode_paged_gqa(*d, scale, num_splits=splits).cpu()
    for b, (i, _) in bad.items():
        rows = np.r_[0:i * bs, (i + 1) * bs:L]
        ref = _oracle(q[b:b + 1], rho[b:b + 1], kc[b:b + 1, :, rows], vc[b:b + 1, :, rows],
                      np.array([len(rows)], np.int32), scale, G)
        check_bf16(o[b:b + 1], ref, f"paged gqa invalid entry b={b} splits={splits}")


def test_paged_gqa_serving_shape():
    """A serving-sized step: B = 8 sequences of up to 4096 rows, 32 query heads over 8 cache
    heads, 256-row blocks, the automatic split plan."""
    B, Hkv, G, L, bs = 8, 8, 4, 4096, 256
    q, rho, kc, vc, sl, scale = _inputs(B, Hkv, G, L, seed=13, rho="proj32")
    kp, vp, table = paginate(kc, vc, sl, bs, seed=17)
    print("paged gqa serving", sl.tolist(), flush=True)
    d = [t.to(DEV) for t in (q, rho, kp, vp, table, sl)]
    o = plx.decode_paged_gqa(*d, scale)
    torch.cuda.synchronize()
    check_bf16(o, _oracle(q, rho, kc, vc, sl, scale, G), "paged gqa serving shape")


@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("bs", [32, 128])
@pytest.mark.parametrize("splits", [0, 3, 8])  # 8: chunks of 128 rows, one step per wave
def test_paged_gqa_d64_equals_contiguous_and_oracle(G, bs, splits):
    """Head dim 64: the paged pool gives the contiguous grouped decode's bits."""
    B, Hkv, L = 3, 2, 1024
    cq = DecodeConfig("pq64", 52, B, Hkv * G, 1, 64, "bf16", "proj32", "full")
    ck = DecodeConfig("pk64", 53, B, Hkv, L, 64, "bf16", "proj32", "uniform_half")
    xq, xk = decode_inputs(cq, seed=G + bs), decode_inputs(ck, seed=G + bs, poison=True)
    q, rho, scale = xq["q"], xq["rho"], xq["scale"]
    kc, vc, sl = xk["k_cache"], xk["v_cache"], xk["seqlens"]
    kp, vp, table = paginate(kc, vc, sl, bs, seed=bs + 3 * G)
    print("paged gqa d64", G, bs, splits, sl.tolist(), flush=True)
    d = [t.to(DEV) for t in (q, rho, kp, vp, table, sl)]
    o = plx.decode_paged_gqa(*d, scale, num_splits=splits)
    s = plx.decode_gqa_plan(B, Hkv * G, Hkv, L, 64, splits)[0]
    ref_c = plx.decode_gqa(d[0], d[1], kc.to(DEV), vc.to(DEV), d[5], scale, num_splits=s)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_c)
    check_bf16(o, _oracle(q, rho, kc, vc, sl, scale, G),
               f"paged gqa d64 G={G} bs={bs} splits={splits}")


@pytest.mark.parametrize("splits", [1, 4, 8])  # 4, 8: one step per wave
def test_paged_gqa_d64_invalid_entry_below_seqlens_is_skipped(splits):
    """Head dim 64, an entry outside [0, num_blocks) inside a sequence's valid range: those
    rows get no weight."""
    B, Hkv, G, L, bs = 3, 2, 4, 512, 64
    cq = DecodeConfig("pq64", 54, B, Hkv * G, 1, 64, "bf16", "proj32", "full")
    ck = DecodeConfig("pk64", 55, B, Hkv, L, 64, "bf16", "proj32", "full")
    xq, xk = decode_inputs(cq, seed=splits), decode_inputs(ck, seed=splits)
    q, rho, scale = xq["q"], xq["rho"], xq["scale"]
    kc, vc, sl = xk["k_cache"], xk["v_cache"], xk["seqlens"]
    kp, vp, table = paginate(kc, vc, sl, bs, seed=19)
    bad = {0: (1, -1), 1: (3, 1 << 30), 2: (0, kp.shape[0])}  # b: (block index, entry)
    for b, (i, entry) in bad.items():
        table[b, i] = entry
    d = [t.to(DEV) for t in (q, rho, kp, vp, table, sl)]
    o = plx.decode_paged_gqa(*d, scale, num_splits=splits).cpu()
    for b, (i, _) in bad.items():
        rows = np.r_[0:i * bs, (i + 1) * bs:L]
        ref = _oracle(q[b:b + 1], rho[b:b + 1], kc[b:b + 1, :, rows], vc[b:b + 1, :, rows],
                      np.array([len(rows)], np.int32), scale, G)
        check_bf16(o[b:b + 1], ref, f"paged gqa d64 invalid entry b={b} splits={splits}")
