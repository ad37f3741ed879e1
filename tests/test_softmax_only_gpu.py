"""GPU parity of the softmax-only specialisation (rho = NULL at the boundary: rho = 0 exactly).

With rho = 0 the method reduces to plain softmax attention (the probe products, P2, O2 and beta
all vanish). The specialised kernels must match the fp64 oracle run with rho = 0, and give the
same bits as the full kernels called with an all-zero rho.
"""
import numpy as np
import pytest
import torch

import attention_plx_attn_amd as plx
import oracle
from parity import check_bf16, check_f32
from plx_synth import decode_inputs, prefill_inputs
from plx_synth.inputs import DecodeConfig, PrefillConfig

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("B,H,T", [(1, 2, 1), (2, 3, 100), (1, 4, 333), (2, 2, 1024)])
def test_prefill_softmax_only_bf16(B, H, T):
    cfg = PrefillConfig("p", 31, B, H, T, 128, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=T)
    _say("prefill softmax-only", B, H, T)
    d = {k: x[k].to(DEV) for k in ("q", "k", "v")}
    o = plx.prefill(d["q"], d["k"], d["v"], None, x["scale"])
    z = plx.prefill(d["q"], d["k"], d["v"], torch.zeros_like(d["q"]), x["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o, z)
    ref = oracle.prefill(x["q"], x["k"], x["v"], np.zeros(x["q"].shape), x["scale"], form="cov")
    check_bf16(o, ref, f"softmax-only prefill B={B} H={H} T={T}")


def test_prefill_softmax_only_f32():
    cfg = PrefillConfig("p", 32, 1, 2, 70, 32, "f32", "proj32")
    x = prefill_inputs(cfg, seed=1)
    d = {k: x[k].to(DEV) for k in ("q", "k", "v")}
    o = plx.prefill(d["q"], d["k"], d["v"], None, x["scale"])
    torch.cuda.synchronize()
    ref = oracle.prefill(x["q"], x["k"], x["v"], np.zeros(x["q"].shape), x["scale"], form="cov")
    check_f32(o, ref, "softmax-only f32")


# split mode (1 and 4 chunks), wave-range mode whole (4 waves) and cut (64 waves)
@pytest.mark.parametrize("splits", [1, 4, -4, -64])
def test_decode_softmax_only(splits):
    cfg = DecodeConfig("d", 33, 5, 4, 700, 128, "bf16", "scaled", "uniform_half")
    x = decode_inputs(cfg, seed=3, poison=True)
    _say("decode softmax-only", splits, x["seqlens"].tolist())
    d = {k: x[k].to(DEV) for k in ("q", "k_cache", "v_cache", "seqlens")}
    o = plx.decode(d["q"], None, d["k_cache"], d["v_cache"], d["seqlens"], x["scale"],
                   num_splits=splits)
    z = plx.decode(d["q"], torch.zeros_like(d["q"]), d["k_cache"], d["v_cache"], d["seqlens"],
                   x["scale"], num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o, z)
    k = torch.nan_to_num(x["k_cache"].float())
    v = torch.nan_to_num(x["v_cache"].float())
    ref = oracle.decode(x["q"], np.zeros(x["q"].shape), k, v, x["seqlens"], x["scale"])
    check_bf16(o, ref, f"softmax-only decode splits={splits}")
