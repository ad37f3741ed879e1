"""GPU parity of the causal prefill kernels against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import attention_plx_attn_amd as plx
import oracle
from parity import (check_bf16, check_f32, metrics, sample_rows, to_f64, ulp_bf16,
                    weight_rounding_bound)
from plx_synth import CONFIGS, prefill_inputs
from plx_synth.inputs import PrefillConfig

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(x, scale=None):
    xd = {k: x[k].to(DEV) for k in ("q", "k", "v", "rho")}
    o = plx.prefill(xd["q"], xd["k"], xd["v"], xd["rho"], x["scale"] if scale is None else scale)
    torch.cuda.synchronize()
    return o


def _say(*a):
    print(*a, flush=True)


def test_tiny_f32_config_all_rows():
    cfg = CONFIGS["tiny_f32"]
    x = prefill_inputs(cfg, seed=0)
    _say("prefill f32", cfg)
    o = _run(x)
    ref = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], x["scale"], form="cov")
    _say(check_f32(o, ref, "tiny_f32"))


@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 5, 64, 65, 150])
def test_f32_head_dims_and_ragged(d, T):
    cfg = PrefillConfig("f32", 11, 2, 3, T, d, "f32", "proj32")
    x = prefill_inputs(cfg, seed=d + T)
    _say("prefill f32", d, T)
    o = _run(x)
    ref = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], x["scale"], form="cov")
    check_f32(o, ref, f"f32 d={d} T={T}")


@pytest.mark.parametrize("T", [1, 2, 31, 64, 65, 127, 128, 129, 200, 257, 384])
def test_bf16_ragged_all_rows(T):
    cfg = PrefillConfig("bf16", 12, 2, 3, T, 128, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=T)
    _say("prefill bf16", T)
    o = _run(x)
    ref = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], x["scale"], form="cov")
    check_bf16(o, ref, f"bf16 T={T}")


def _check_stress(o, x, ref, what):
    """Stress inputs beyond the workload recipes: rel-L2 at the bf16 bar, every element
    within half an output ulp + 1e-3 + the derived weight-rounding bound."""
    m = metrics(o, ref)
    _say(what, m)
    assert m["finite"] and m["rel_l2"] <= 5e-3, m
    bound = weight_rounding_bound(x["q"], x["k"], x["v"], x["rho"], x["scale"])
    err = np.abs(to_f64(o) - ref)
    assert (err <= 0.5 * ulp_bf16(ref) + 1e-3 + bound).all(), float((err - bound).max())


def test_bf16_wide_scores_within_derived_rounding_bound():
    # q scaled x3: a sharper softmax (fewer keys average the weight roundings) whose
    # scores spread well past the lazy-rescale threshold of the running max.
    cfg = PrefillConfig("bf16", 13, 1, 4, 300, 128, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=1)
    x["q"] = (x["q"].float() * 3).to(torch.bfloat16)
    o = _run(x)
    ref = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], x["scale"], form="cov")
    _check_stress(o, x, ref, "wide scores")


def test_bf16_strong_probe_within_derived_rounding_bound():
    # Unit-RMS probe (|t| up to ~40, ten times the workload probes): bf16 rounding of
    # w*t dominates the error.
    cfg = PrefillConfig("bf16", 13, 1, 4, 300, 128, "bf16", "proj32")
    x = prefill_inputs(cfg, seed=1)
    o = _run(x)
    ref = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], x["scale"], form="cov")
    _check_stress(o, x, ref, "strong probe")


def test_bf16_scale_zero_uniform_weights():
    cfg = PrefillConfig("bf16", 14, 1, 2, 140, 128, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=2)
    o = _run(x, scale=0.0)
    ref = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], 0.0, form="cov")
    check_bf16(o, ref, "scale 0")


def test_bf16_first_row_is_first_value_bitwise():
    cfg = PrefillConfig("bf16", 15, 2, 4, 96, 128, "bf16", "proj32")
    x = prefill_inputs(cfg, seed=3)
    o = _run(x).cpu()
    assert torch.equal(o[:, :, 0], x["v"][:, :, 0])


def test_bf16_rho_zero_heads_are_softmax_and_independent():
    cfg = PrefillConfig("bf16", 16, 1, 4, 200, 128, "bf16", "half_zero_heads")
    x = prefill_inputs(cfg, seed=4)
    o = _run(x).cpu()
    # zero-probe heads equal plain softmax attention (torch SDPA in fp64 on the CPU)
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        x["q"][:, :2].double(), x["k"][:, :2].double(), x["v"][:, :2].double(), is_causal=True,
        scale=x["scale"])
    check_bf16(o[:, :2], sdpa, "rho=0 vs SDPA")
    # ... and are bitwise independent of the other heads' probes
    x2 = dict(x)
    x2["rho"] = torch.zeros_like(x["rho"])
    o2 = _run(x2).cpu()
    assert torch.equal(o[:, :2], o2[:, :2])


def test_bf16_future_keys_do_not_leak():
    cfg = PrefillConfig("bf16", 17, 1, 2, 256, 128, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=5)
    o1 = _run(x).cpu()
    cut = 100
    x2 = dict(x)
    for name in ("k", "v"):
        t = x[name].clone()
        t[:, :, cut + 1:] = torch.randn_like(t[:, :, cut + 1:].float()).to(t.dtype) * 5
        x2[name] = t
    o2 = _run(x2).cpu()
    assert torch.equal(o1[:, :, : cut + 1], o2[:, :, : cut + 1])
    assert not torch.equal(o1[:, :, cut + 1:], o2[:, :, cut + 1:])


def test_bf16_deterministic():
    cfg = PrefillConfig("bf16", 18, 2, 2, 333, 128, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=6)
    assert torch.equal(_run(x), _run(x))


def test_bf16_batch_permutation_equivariance():
    cfg = PrefillConfig("bf16", 19, 3, 2, 130, 128, "bf16", "scaled")
    x = prefill_inputs(cfg, seed=7)
    o = _run(x).cpu()
    perm = torch.tensor([2, 0, 1])
    xp = {k: (x[k][perm] if k != "scale" else x[k]) for k in x}
    op = _run(xp).cpu()
    assert torch.equal(op, o[perm])


def test_bf16_config_prefill_4x16x2048_full():
    cfg = CONFIGS["prefill_bf16"]
    _say("prefill bf16 full config", cfg)
    x = prefill_inputs(cfg, seed=0)
    o = _run(x)
    ref = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], x["scale"], form="sweighted")
    _say("all rows (corrected-weight form)", check_bf16(o, ref, "prefill_bf16 all rows"))
    rows = sample_rows(cfg.B, cfg.H, cfg.T, n_random=8)
    refc = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], x["scale"], form="cov", rows=rows)
    got = o.reshape(-1, cfg.d)[torch.from_numpy(rows).to(DEV)]
    _say("sampled rows (definition)", check_bf16(got, refc, "prefill_bf16 sampled"))


def test_bf16_config_prefill_long_1x32x32768():
    cfg = CONFIGS["prefill_long"]
    _say("prefill bf16 long config", cfg)
    x = prefill_inputs(cfg, seed=0)
    o = _run(x)
    rows = sample_rows(cfg.B, cfg.H, cfg.T, n_random=16, seed=1)
    ref = oracle.prefill(x["q"], x["k"], x["v"], x["rho"], x["scale"], form="sweighted",
                         rows=rows)
    got = o.reshape(-1, cfg.d)[torch.from_numpy(rows).to(DEV)]
    half = (rows // cfg.T) < cfg.H // 2
    _say("zero-probe heads", check_bf16(got[torch.from_numpy(half).to(DEV)], ref[half], "rho=0"))
    _say("probe heads", check_bf16(got[torch.from_numpy(~half).to(DEV)], ref[~half], "rho!=0"))
    # zero-probe heads: same bits as a run where every head has rho = 0
    x0 = dict(x)
    x0["rho"] = torch.zeros_like(x["rho"])
    o0 = _run(x0)
    assert torch.equal(o[:, : cfg.H // 2], o0[:, : cfg.H // 2])
