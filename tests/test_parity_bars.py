"""The gradient bar admits what the backward kernels' own roundings produce (CPU).

tests/parity.py::backward_rounding_emulation is the causal prefill backward in fp64 with the
kernels' rounding points (the forward's bf16 vbar and o; the pair quantities s, scale * da and
dt in bf16 before their products). A kernel that rounds exactly there and sums exactly would
produce these gradients; rounded to bf16 like the kernels' outputs they must pass check_grad
against the oracle, or the bar would fail a correct kernel.
"""
import numpy as np
import pytest

import oracle
from parity import _bf16, backward_rounding_emulation, check_grad, to_f64
from plx_synth import prefill_inputs, prefill_upstream_grad
from plx_synth.inputs import PrefillConfig


@pytest.mark.parametrize("B,H,T,d,rho", [(1, 2, 31, 128, "proj32"), (1, 2, 64, 128, "proj32"),
                                         (1, 2, 100, 64, "scaled"), (1, 1, 300, 128, "zero"),
                                         (1, 2, 130, 128, "scaled")])
def test_emulated_backward_roundings_pass_the_gradient_bar(B, H, T, d, rho):
    cfg = PrefillConfig("bwd", 43, B, H, T, d, "bf16", rho)
    x = prefill_inputs(cfg, seed=T + 1)
    do = to_f64(prefill_upstream_grad(cfg, seed=T + 1))
    f = [to_f64(x[n]) for n in ("q", "k", "v", "rho")]
    ref = oracle.prefill_backward(*f, x["scale"], do)
    emu = backward_rounding_emulation(*f, x["scale"], do)
    for name, e, r in zip(("dq", "dk", "dv", "drho"), emu, ref):
        if np.any(r):
            check_grad(_bf16(e), r, f"emulated {name}")


def test_emulation_without_roundings_is_the_oracle():
    # Apart from its bf16 roundings the emulation is the chain rule of the forward: it must
    # agree with the oracle's backward to rel-L2 below 1e-2, which a dropped term or a wrong
    # sign in it would break.
    cfg = PrefillConfig("bwd", 47, 1, 1, 40, 16, "f32", "proj32")
    x = prefill_inputs(cfg, seed=0)
    do = to_f64(prefill_upstream_grad(cfg, seed=0))
    f = [to_f64(x[n]) for n in ("q", "k", "v", "rho")]
    ref = oracle.prefill_backward(*f, x["scale"], do)
    emu = backward_rounding_emulation(*f, x["scale"], do)
    for e, r in zip(emu, ref):
        assert np.linalg.norm(e - r) <= 1e-2 * np.linalg.norm(r)
