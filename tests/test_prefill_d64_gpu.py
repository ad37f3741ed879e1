"""GPU parity of the bf16 prefill at head dim 64 (the compute-matched head dim: halving d makes
a Parallax layer's four pair products cost what softmax attention's two cost at d = 128) against
the fp64 oracle, with the structure checks of the d = 128 kernel."""
import numpy as np
import pytest
import torch

import attention_plx_attn_amd as plx
import oracle
from parity import check_bf16, metrics, to_f64, ulp_bf16, weight_rounding_bound
from plx_synth import prefill_inputs
from plx_synth.inputs import PrefillConfig

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _run(x, rho=True, split=False):
    d = {k: x[k].to(DEV) for k in ("q", "k", "v", "rho")}
    o = plx.prefill(d["q"], d["k"], d["v"], d["rho"] if rho else None, x["scale"],
                    split_weights=split)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("B,H,T", [(1, 2, 1), (2, 3, 31), (1, 2, 64), (2, 3, 100),
                                   (1, 4, 333), (2, 2, 1024)])
def test_d64_parity(B, H, T):
    cfg = PrefillConfig("d64", 51, B, H, T, 64, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=T)
    _say("prefill d64", B, H, T)
    o = _run(x)
    ref = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], x["scale"], form="cov")
    _say(check_bf16(o, ref, f"d64 B={B} H={H} T={T}"))


@pytest.mark.parametrize("B,H,T", [(1, 2, 1), (2, 3, 31), (1, 4, 333), (2, 2, 1024)])
def test_d64_split_parity(B, H, T):
    cfg = PrefillConfig("d64", 51, B, H, T, 64, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=T)
    o = _run(x, split=True)
    ref = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], x["scale"], form="cov")
    _say(check_bf16(o, ref, f"d64 split B={B} H={H} T={T}"))


@pytest.mark.parametrize("qs", [1, 3])
@pytest.mark.parametrize("T", [31, 300])
def test_d64_strong_probe(T, qs):
    # Unit-RMS probe (|t| ~ 8 at d = 64, ten times the workload probes): split weights meet the
    # plain bf16 bar; single bf16 weights keep rel-L2 at the bar and every element within half
    # an output ulp + 1e-3 + the first-order weight-rounding bound.
    cfg = PrefillConfig("d64", 55, 2, 3, T, 64, "bf16", "proj32")
    x = prefill_inputs(cfg, seed=T)
    x["q"] = (x["q"].float() * qs).to(torch.bfloat16)
    ref = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], x["scale"], form="cov")
    ms = check_bf16(_run(x, split=True), ref, f"d64 strong probe split T={T} q*{qs}")
    o = _run(x)
    m = metrics(o, ref)
    _say(f"STRESS d=64 T={T} rms=1(proj32) q*{qs}: default excess "
         f"{m['excess_over_half_ulp']:.4f} rel {m['rel_l2']:.2e} | split excess "
         f"{ms['excess_over_half_ulp']:.4f} rel {ms['rel_l2']:.2e}")
    assert m["finite"] and m["rel_l2"] <= 5e-3, m
    bound = weight_rounding_bound(x["q"], x["k"], x["v"], x["rho"], x["scale"])
    err = np.abs(to_f64(o) - ref)
    assert (err <= 0.5 * ulp_bf16(ref) + 1e-3 + bound).all(), float((err - bound).max())


def test_d64_softmax_only_is_rho_zero_bitwise():
    cfg = PrefillConfig("d64", 52, 2, 2, 300, 64, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=1)
    o = _run(x, rho=False)
    x0 = dict(x)
    x0["rho"] = torch.zeros_like(x["rho"])
    assert torch.equal(o, _run(x0))
    ref = oracle.prefill(x["q"], x["k"], x["v"], np.zeros(x["q"].shape), x["scale"], form="cov")
    check_bf16(o, ref, "d64 softmax only")


def test_d64_structure():
    cfg = PrefillConfig("d64", 53, 2, 2, 256, 64, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=2)
    o1 = _run(x).cpu()
    assert torch.equal(o1[:, :, 0], x["v"][:, :, 0])        # row 0 is v_0
    assert torch.equal(o1, _run(x).cpu())                   # deterministic
    cut = 100
    x2 = dict(x)
    for name in ("k", "v"):
        t = x[name].clone()
        t[:, :, cut + 1:] = (torch.randn_like(t[:, :, cut + 1:].float()) * 5).to(t.dtype)
        x2[name] = t
    o2 = _run(x2).cpu()
    assert torch.equal(o1[:, :, : cut + 1], o2[:, :, : cut + 1])   # no future key leaks


def test_d64_full_size_sampled_rows():
    """B=4, H=32, T=2048, d=64: the compute-matched counterpart of the prefill workload (twice
    the heads at half the head dim); every row of three sampled (b, h)."""
    cfg = PrefillConfig("d64_full", 54, 4, 32, 2048, 64, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=0)
    _say("prefill d64 full", cfg)
    o = _run(x)
    for b, h in ((0, 0), (2, 17), (3, 31)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.prefill(x["q"][sl], x["k"][sl], x["v"][sl], x["rho"][sl], x["scale"],
                             form="cov")
        check_bf16(o[sl], ref, f"d64 full b={b} h={h}")
