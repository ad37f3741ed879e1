"""The seeded workload generators: determinism, shapes, recipes."""
import numpy as np
import torch

from plx_synth import CONFIGS, decode_grid_cells, decode_inputs, prefill_inputs
from plx_synth.inputs import DecodeConfig, PrefillConfig, draw_seqlens


def test_configs_present():
    assert CONFIGS["tiny_f32"].T == 64 and CONFIGS["tiny_f32"].d == 16
    assert CONFIGS["prefill_bf16"].B == 4 and CONFIGS["prefill_bf16"].T == 2048
    assert CONFIGS["decode_32k"].L_max == 32768
    assert CONFIGS["prefill_long"].T == 32768 and CONFIGS["prefill_long"].H == 32
    cells = decode_grid_cells()
    assert len(cells) == 18
    assert all(c.B * c.L_max <= (1 << 23) for c in cells)


def test_prefill_deterministic_and_dtypes():
    cfg = CONFIGS["tiny_f32"]
    a = prefill_inputs(cfg, seed=3)
    b = prefill_inputs(cfg, seed=3)
    c = prefill_inputs(cfg, seed=4)
    for n in ("q", "k", "v", "rho"):
        assert a[n].dtype == torch.float32 and a[n].shape == (1, 2, 64, 16)
        assert torch.equal(a[n], b[n])
        assert not torch.equal(a[n], c[n])
    # proj32 probe: RMSNorm per head -> unit RMS over d
    rms = a["rho"].double().pow(2).mean(-1).sqrt()
    np.testing.assert_allclose(rms.numpy(), 1.0, atol=1e-4)  # eps = 1e-6 inside the norm
    assert abs(a["scale"] - 0.25) < 1e-15


def test_bf16_scaled_rho_and_half_zero_heads():
    cfg = PrefillConfig("t", 5, 1, 4, 32, 128, "bf16", "half_zero_heads")
    x = prefill_inputs(cfg, seed=0)
    assert x["q"].dtype == torch.bfloat16
    assert torch.all(x["rho"][:, :2] == 0)
    rms = x["rho"][:, 2:].double().pow(2).mean(-1).sqrt()
    np.testing.assert_allclose(rms.numpy(), 0.1, rtol=1e-2)


def test_decode_seqlens_and_poison():
    cfg = DecodeConfig("t", 4, 16, 2, 64, 16, "bf16", "scaled", "uniform_half")
    sl = draw_seqlens(cfg, seed=1)
    assert sl.min() >= 32 and sl.max() <= 64
    x = decode_inputs(cfg, seed=1, poison=True)
    for b in range(cfg.B):
        n = int(sl[b])
        assert torch.isnan(x["k_cache"][b, :, n:].float()).all()
        assert not torch.isnan(x["k_cache"][b, :, :n].float()).any()


def test_chunks_regenerate_independently():
    # Batch row b of a larger workload equals the same row drawn alone.
    big = DecodeConfig("t", 7, 3, 2, 40, 8, "f32", "scaled", "full")
    x = decode_inputs(big, seed=9)
    for b in range(3):
        assert torch.isfinite(x["k_cache"][b]).all()
    y = decode_inputs(DecodeConfig("t", 7, 3, 2, 40, 8, "f32", "scaled", "full"), seed=9)
    assert torch.equal(x["v_cache"], y["v_cache"])


def test_prefill_head_inputs_equal_the_full_draw_slice():
    from plx_synth import prefill_head_inputs
    cfg = PrefillConfig("t", 5, 2, 4, 40, 128, "bf16", "half_zero_heads")
    full = prefill_inputs(cfg, seed=2)
    for b, h in ((0, 0), (1, 1), (0, 2), (1, 3)):
        one = prefill_head_inputs(cfg, b, h, seed=2)
        for n in ("q", "k", "v", "rho"):
            assert torch.equal(one[n], full[n][b: b + 1, h: h + 1]), (b, h, n)
