"""GPU parity of the paged-cache decode (plx_attn_decode_paged).

A contiguous cache is scattered into a pool of blocks in a random order; the paged call must
give the same bits as the contiguous split decode with the same split count (the arithmetic
is identical), and match the fp64 oracle on the contiguous cache. Table entries past each
sequence's last block hold garbage that must never be used.
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


def _paged(x, bs, seed):
    kc, vc, sl = x["k_cache"], x["v_cache"], x["seqlens"]
    B, H, L, d = kc.shape
    mb = L // bs
    rng = np.random.default_rng(seed)
    nblk = B * mb + 3
    perm = rng.permutation(nblk)[: B * mb].reshape(B, mb)
    kp = torch.full((nblk, H, bs, d), float("nan"), dtype=kc.dtype)
    vp = torch.full((nblk, H, bs, d), float("nan"), dtype=vc.dtype)
    table = torch.from_numpy(perm.astype(np.int32)).clone()
    for b in range(B):
        n = int(sl[b])
        used = (n + bs - 1) // bs
        for i in range(mb):
            if i < used:
                kp[perm[b, i]] = kc[b, :, i * bs:(i + 1) * bs]
                vp[perm[b, i]] = vc[b, :, i * bs:(i + 1) * bs]
            else:
                table[b, i] = [-7, 1 << 30, nblk][i % 3]   # never dereferenced
    return kp, vp, table


@pytest.mark.parametrize("bs", [32, 64, 256])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_paged_equals_contiguous_and_oracle(bs, splits):
    cfg = DecodeConfig("d", 42, 4, 3, 1024, 128, "bf16", "scaled", "uniform_half")
    x = decode_inputs(cfg, seed=bs + splits, poison=True)
    kp, vp, table = _paged(x, bs, seed=bs)
    print("paged", bs, splits, x["seqlens"].tolist(), flush=True)
    q, rho, sl = (x[k].to(DEV) for k in ("q", "rho", "seqlens"))
    o = plx.decode_paged(q, rho, kp.to(DEV), vp.to(DEV), table.to(DEV), sl, x["scale"],
                         num_splits=splits)
    s = plx.decode_gqa_plan(4, 3, 3, 1024, 128, splits)[0]
    ref_c = plx.decode(q, rho, x["k_cache"].to(DEV), x["v_cache"].to(DEV), sl, x["scale"],
                       num_splits=s)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_c)
    k = torch.nan_to_num(x["k_cache"].float())
    v = torch.nan_to_num(x["v_cache"].float())
    ref = oracle.decode(x["q"], x["rho"], k, v, x["seqlens"], x["scale"], form="cov")
    check_bf16(o, ref, f"paged bs={bs} splits={splits}")


def test_paged_seqlens_edges_and_softmax_only():
    cfg = DecodeConfig("d", 43, 5, 2, 256, 128, "bf16", "scaled", "full")
    x = decode_inputs(cfg, seed=4)
    sl = torch.tensor([0, -2, 1, 256, 999], dtype=torch.int32)
    x["seqlens"] = sl
    kp, vp, table = _paged(x, 64, seed=5)
    d = [t.to(DEV) for t in (x["q"], x["rho"], kp, vp, table, sl)]
    o = plx.decode_paged(d[0], d[1], d[2], d[3], d[4], d[5], x["scale"], num_splits=2).cpu()
    z = plx.decode_paged(d[0], None, d[2], d[3], d[4], d[5], x["scale"], num_splits=2).cpu()
    z0 = plx.decode_paged(d[0], torch.zeros_like(d[1]), d[2], d[3], d[4], d[5], x["scale"],
                          num_splits=2).cpu()
    assert torch.equal(z, z0)
    assert torch.all(o[0] == 0) and torch.all(o[1] == 0)
    assert torch.equal(o[2], x["v_cache"][2, :, 0])
    ref = oracle.decode(x["q"], x["rho"], x["k_cache"], x["v_cache"], sl, x["scale"])
    check_bf16(o[3:], ref[3:], "paged edges")
