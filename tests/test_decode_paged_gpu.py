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
from paged_cache import paginate
from parity import check_bf16
from plx_synth import decode_inputs
from plx_synth.inputs import DecodeConfig

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _paged(x, bs, seed):
    return paginate(x["k_cache"], x["v_cache"], x["seqlens"], bs, seed)


@pytest.mark.parametrize("rho_kind", ["scaled", "proj32"])
@pytest.mark.parametrize("bs", [32, 64, 256])
@pytest.mark.parametrize("splits", [0, 1, 3, 8])  # 8: chunks of 128 rows, one step per wave
def test_paged_equals_contiguous_and_oracle(bs, splits, rho_kind):
    cfg = DecodeConfig("d", 42, 4, 3, 1024, 128, "bf16", rho_kind, "uniform_half")
    x = decode_inputs(cfg, seed=bs + splits, poison=True)
    kp, vp, table = _paged(x, bs, seed=bs)
    print("paged", bs, splits, rho_kind, x["seqlens"].tolist(), flush=True)
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
    check_bf16(o, ref, f"paged bs={bs} splits={splits} rho={rho_kind}")


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


@pytest.mark.parametrize("splits", [1, 3, 4, 8])  # 4, 8: one step per wave
def test_paged_invalid_entry_below_seqlens_is_skipped(splits):
    """A table entry outside [0, num_blocks) inside a sequence's valid range: those rows get
    no weight, so the output equals the oracle over the sequence without them."""
    bs = 64
    cfg = DecodeConfig("d", 44, 3, 2, 512, 128, "bf16", "proj32", "full")
    x = decode_inputs(cfg, seed=6)
    kp, vp, table = _paged(x, bs, seed=7)
    bad = {0: (1, -1), 1: (3, 1 << 30), 2: (0, kp.shape[0])}  # b: (block index, entry)
    keep = []
    for b, (i, entry) in bad.items():
        table[b, i] = entry
        rows = np.r_[0:i * bs, (i + 1) * bs:512]
        keep.append(rows)
    d = [t.to(DEV) for t in (x["q"], x["rho"], kp, vp, table, x["seqlens"])]
    o = plx.decode_paged(*d, x["scale"], num_splits=splits).cpu()
    for b, rows in enumerate(keep):
        k = x["k_cache"][b: b + 1, :, rows]
        v = x["v_cache"][b: b + 1, :, rows]
        ref = oracle.decode(x["q"][b: b + 1], x["rho"][b: b + 1], k, v,
                            np.array([len(rows)], np.int32), x["scale"])
        check_bf16(o[b: b + 1], ref, f"paged invalid entry b={b} splits={splits}")


@pytest.mark.parametrize("bs", [32, 256])
@pytest.mark.parametrize("splits", [0, 3, 8])  # 8: one step per wave
def test_paged_d64_equals_grouped_and_oracle(bs, splits):
    """Head dim 64: the paged decode runs the grouped kernel with one query head per cache
    head, so it gives plx_attn_decode_gqa's bits on the contiguous cache."""
    cfg = DecodeConfig("d64", 45, 4, 3, 1024, 64, "bf16", "proj32", "uniform_half")
    x = decode_inputs(cfg, seed=bs + splits, poison=True)
    kp, vp, table = _paged(x, bs, seed=bs + 1)
    print("paged d64", bs, splits, x["seqlens"].tolist(), flush=True)
    q, rho, sl = (x[k].to(DEV) for k in ("q", "rho", "seqlens"))
    o = plx.decode_paged(q, rho, kp.to(DEV), vp.to(DEV), table.to(DEV), sl, x["scale"],
                         num_splits=splits)
    s = plx.decode_gqa_plan(4, 3, 3, 1024, 64, splits)[0]
    ref_c = plx.decode_gqa(q, rho, x["k_cache"].to(DEV), x["v_cache"].to(DEV), sl, x["scale"],
                           num_splits=s)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_c)
    k = torch.nan_to_num(x["k_cache"].float())
    v = torch.nan_to_num(x["v_cache"].float())
    ref = oracle.decode(x["q"], x["rho"], k, v, x["seqlens"], x["scale"], form="cov")
    check_bf16(o, ref, f"paged d64 bs={bs} splits={splits}")
