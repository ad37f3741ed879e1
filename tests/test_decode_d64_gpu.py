"""GPU parity of the decode step at head dim 64 (the compute-matched head dim; split-KV partials
and their combine) against the fp64 oracle, with the d = 128 decode's structure checks."""
import numpy as np
import pytest
import torch

import attention_plx_attn_amd as plx
import oracle
from parity import check_bf16
from plx_synth import decode_inputs
from plx_synth.inputs import DecodeConfig, PrefillConfig, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _run(x, num_splits=0, seqlens=None, rho=True):
    sl = (x["seqlens"] if seqlens is None else seqlens).to(DEV)
    o = plx.decode(x["q"].to(DEV), x["rho"].to(DEV) if rho else None, x["k_cache"].to(DEV),
                   x["v_cache"].to(DEV), sl, x["scale"], num_splits=num_splits)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("rho", ["scaled", "proj32"])
@pytest.mark.parametrize("splits", [0, 1, 3, 16])
@pytest.mark.parametrize("L", [1, 40, 300, 1000])
def test_d64_decode_with_poisoned_tail(L, splits, rho):
    cfg = DecodeConfig("d64", 61, 3, 4, L, 64, "bf16", rho, "uniform_half")
    x = decode_inputs(cfg, seed=L, poison=True)
    _say("decode d64", L, splits, rho, x["seqlens"].tolist())
    o = _run(x, splits)
    k = torch.nan_to_num(x["k_cache"].float())  # rows >= seqlens are never read
    v = torch.nan_to_num(x["v_cache"].float())
    ref = oracle.decode(x["q"], x["rho"], k, v, x["seqlens"], x["scale"], form="cov")
    check_bf16(o, ref, f"d64 L={L} splits={splits} rho={rho}")


@pytest.mark.parametrize("rho", ["scaled", "proj32"])
def test_d64_seqlens_edge_cases(rho):
    cfg = DecodeConfig("d64", 62, 5, 2, 200, 64, "bf16", rho, "full")
    x = decode_inputs(cfg, seed=1)
    sl = torch.tensor([0, -5, 1, 200, 100000], dtype=torch.int32)
    for splits in (1, 4):
        o = _run(x, splits, seqlens=sl).cpu()
        assert torch.all(o[0] == 0) and torch.all(o[1] == 0)
        assert torch.equal(o[2], x["v_cache"][2, :, 0])  # one key: exactly its value
        ref = oracle.decode(x["q"], x["rho"], x["k_cache"], x["v_cache"], sl, x["scale"])
        check_bf16(o[3:], ref[3:], f"d64 edges splits={splits}")


def test_d64_softmax_only_is_rho_zero_bitwise():
    cfg = DecodeConfig("d64", 63, 4, 3, 700, 64, "bf16", "scaled", "uniform_half")
    x = decode_inputs(cfg, seed=2)
    for splits in (1, 5):
        o = _run(x, splits, rho=False)
        x0 = dict(x)
        x0["rho"] = torch.zeros_like(x["rho"])
        assert torch.equal(o, _run(x0, splits))
        ref = oracle.decode(x["q"], np.zeros(x["q"].shape), x["k_cache"], x["v_cache"],
                            x["seqlens"], x["scale"])
        check_bf16(o, ref, f"d64 softmax only splits={splits}")


def test_d64_decode_equals_last_prefill_row_and_is_deterministic():
    p = prefill_inputs(PrefillConfig("p", 64, 2, 2, 333, 64, "bf16", "scaled"), seed=3)
    pd = {k: p[k].to(DEV) for k in ("q", "k", "v", "rho")}
    pre = plx.prefill(pd["q"], pd["k"], pd["v"], pd["rho"], p["scale"]).cpu()
    sl = torch.full((2,), 333, dtype=torch.int32, device=DEV)
    call = lambda: plx.decode(pd["q"][:, :, -1].contiguous(), pd["rho"][:, :, -1].contiguous(),  # noqa: E731
                              pd["k"], pd["v"], sl, p["scale"], num_splits=3).cpu()
    dec = call()
    assert torch.equal(dec, call())
    ref = oracle.decode(p["q"][:, :, -1], p["rho"][:, :, -1], p["k"], p["v"], sl.cpu(),
                        p["scale"])
    check_bf16(dec, ref, "d64 decode")
    check_bf16(pre[:, :, -1], ref, "d64 prefill last row")


def test_d64_long_cache_auto_plan():
    """B=1, H=16, one 32768-row cache at d = 64 (the decode workload at the halved head dim),
    automatic split plan, every output row against the oracle."""
    cfg = DecodeConfig("d64_long", 65, 1, 16, 32768, 64, "bf16", "proj32", "full")
    x = decode_inputs(cfg, seed=0)
    _say("decode d64 long", plx.decode_num_splits(1, 16, 32768, 0))
    o = _run(x, 0)
    ref = oracle.decode(x["q"], x["rho"], x["k_cache"], x["v_cache"], x["seqlens"], x["scale"])
    check_bf16(o, ref, "d64 long")
