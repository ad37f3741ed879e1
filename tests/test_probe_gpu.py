"""GPU parity of the probe producer (plx_attn_probe) against the fp64 oracle.probe.

Inputs follow the configs' probe recipe: x ~ N(0, 1) rows of width C, W_R ~ N(0, 0.05^2),
rounded to bf16 once; the oracle reads the same bf16 values widened to fp64.
"""
import numpy as np
import pytest
import torch

import attention_plx_attn_amd as plx
import oracle
from parity import check_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(seed, B, T, C, H, d=128):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((B, T, C))).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((H * d, C)) * 0.05).to(torch.bfloat16)
    gamma = torch.from_numpy(1.0 + 0.2 * rng.standard_normal(d)).float()
    gate = torch.from_numpy(1.0 / (1.0 + np.exp(-rng.standard_normal(H)))).float()
    return x, w, gamma, gate


# (B, T, C, H): decode-like single tokens; ragged token counts (not a multiple of 64);
# an input width that is not a multiple of 32; a wide input (many K steps); the widths on either
# side of the switch from one to two token groups per wave (64 / 96); two heads per workgroup
# (one K step, even H) with 16-token groups inside one sequence (T = 160) and across
# sequence ends (T = 77), and the odd-H and two-K-step cases that keep one head
@pytest.mark.parametrize("B,T,C,H", [(4, 1, 32, 16), (2, 100, 32, 3), (3, 77, 40, 2),
                                     (1, 64, 2048, 2), (1, 300, 256, 1), (2, 130, 64, 2),
                                     (1, 129, 96, 2), (2, 160, 32, 4), (3, 77, 24, 2)])
@pytest.mark.parametrize("opts", ["plain", "gamma_gate", "rope"])
def test_probe_matches_oracle(B, T, C, H, opts):
    x, w, gamma, gate = _inputs(B * 1000 + T + C, B, T, C, H)
    kw, kwo = {}, {}
    if opts == "gamma_gate":
        kw = {"gamma": gamma.to(DEV), "gate": gate.to(DEV)}
        kwo = {"gamma": gamma.numpy(), "gate": gate.numpy()}
    if opts == "rope":
        pos = torch.arange(B, dtype=torch.int32) * 1000 + 17
        kw = {"rope_base": 10000.0, "positions": pos.to(DEV)}
        kwo = {"rope_base": 10000.0, "positions": pos.numpy()}
    print("probe", B, T, C, H, opts, flush=True)
    rho = plx.probe(x.to(DEV), w.to(DEV), H, eps=1e-6, **kw)
    torch.cuda.synchronize()
    ref = oracle.probe(x.float().numpy(), w.float().numpy(), H, eps=1e-6, **kwo)
    check_bf16(rho, ref, f"probe B={B} T={T} C={C} H={H} {opts}")


def test_probe_zero_projection_and_decode_positions():
    B, H, C = 5, 4, 32
    x, w, _, _ = _inputs(7, B, 1, C, H)
    rho = plx.probe(x.to(DEV), torch.zeros_like(w).to(DEV), H, eps=1e-6)
    torch.cuda.synchronize()
    assert torch.all(rho == 0)
    # one decode token per sequence at position seqlens[b] - 1
    sl = torch.tensor([1, 9, 32768, 4000, 2], dtype=torch.int32)
    rho = plx.probe(x.to(DEV), w.to(DEV), H, eps=1e-6, rope_base=10000.0,
                    positions=(sl - 1).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.probe(x.float().numpy(), w.float().numpy(), H, eps=1e-6, rope_base=10000.0,
                       positions=(sl - 1).numpy())
    check_bf16(rho, ref, "decode positions")
