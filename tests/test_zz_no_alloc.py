"""plx_attn_decode_noalloc (split records in the library's fixed per-GPU scratch, nothing
allocated by the call) against plx_attn_decode with a caller workspace, through the C ABI.

Both run the same plan and kernels, so their outputs must have the same bits; each is also
checked against the fp64 oracle. Two calls in a row, the second with a smaller input, show
that what the first left in the shared scratch does not leak into the second.
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


def _say(*a):
    print(*a, flush=True)


def _dev(x):
    return {k: x[k].to(DEV) for k in ("q", "rho", "k_cache", "v_cache", "seqlens")}


def _both(x, splits):
    g = _dev(x)
    ref = plx.decode(g["q"], g["rho"], g["k_cache"], g["v_cache"], g["seqlens"], x["scale"],
                     num_splits=splits)
    out = torch.full_like(ref, float("nan"))
    got = plx.decode_noalloc(g["q"], g["rho"], g["k_cache"], g["v_cache"], g["seqlens"], out,
                             x["scale"], num_splits=splits)
    torch.cuda.synchronize()
    return got.cpu(), ref.cpu()


def _oracle(x):
    k = torch.nan_to_num(x["k_cache"].float())
    v = torch.nan_to_num(x["v_cache"].float())
    return oracle.decode(x["q"], x["rho"], k, v, x["seqlens"], x["scale"])


@pytest.mark.parametrize("splits", [16, 0, -64])
def test_noalloc_equals_decode_on_two_calls_second_smaller(splits):
    big = decode_inputs(DecodeConfig("na", 71, 2, 16, 4096, 128, "bf16", "proj32",
                                     "uniform_half"), seed=1, poison=True)
    small = decode_inputs(DecodeConfig("na", 72, 1, 3, 300, 128, "bf16", "proj32",
                                       "uniform_half"), seed=2, poison=True)
    for name, x, s in (("first (larger)", big, splits), ("second (smaller)", small,
                                                         splits if splits <= 0 else 3)):
        _say("noalloc", name, "splits", s, "plan", plx.decode_num_splits(
            *x["k_cache"].shape[:3], s), "workspace", plx.decode_workspace_size(
            *x["k_cache"].shape[:3], 128, s))
        got, ref = _both(x, s)
        assert torch.equal(got, ref), name
        _say(name, check_bf16(got, _oracle(x), f"noalloc {name}"))


def test_noalloc_d64_and_softmax_only():
    x = decode_inputs(DecodeConfig("na", 73, 2, 4, 2000, 64, "bf16", "proj32", "uniform_half"),
                      seed=3)
    got, ref = _both(x, 5)
    assert torch.equal(got, ref)
    check_bf16(got, _oracle(x), "noalloc d64")
    g = _dev(x)
    out = torch.empty_like(g["q"])
    z = plx.decode_noalloc(g["q"], None, g["k_cache"], g["v_cache"], g["seqlens"], out,
                           x["scale"], num_splits=5)
    z0 = plx.decode(g["q"], torch.zeros_like(g["rho"]), g["k_cache"], g["v_cache"],
                    g["seqlens"], x["scale"], num_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(z, z0)


def test_noalloc_rejects_plans_beyond_the_scratch():
    # 2 x 16 (b, h) x 512 chunks (4096 requested; 64-row chunks of 32768) x 1040-byte records
    # = 17.0 MB > 16 MiB: rejected before anything is enqueued (the cache values are unused)
    B, H, L, d = 2, 16, 32768, 128
    assert plx.decode_workspace_size(B, H, L, d, 4096) > (16 << 20)
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((B, H, L, d), dtype=torch.bfloat16, device=DEV)
    sl = torch.full((B,), L, dtype=torch.int32, device=DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(plx.PlxError) as e:
        plx.decode_noalloc(q, q, kc, kc, sl, out, None, num_splits=4096)
    assert e.value.code == 6  # PLX_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
