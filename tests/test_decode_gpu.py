"""GPU parity of the decode kernels (split partials + combine) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import attention_plx_attn_amd as plx
import oracle
from parity import check_bf16
from plx_synth import CONFIGS, decode_grid_cells, decode_inputs
from plx_synth.inputs import DecodeConfig, host_draw_ok

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _run(x, num_splits=0, scale=None, seqlens=None):
    sl = (x["seqlens"] if seqlens is None else seqlens).to(DEV)
    o = plx.decode(x["q"].to(DEV), x["rho"].to(DEV), x["k_cache"].to(DEV),
                   x["v_cache"].to(DEV), sl, x["scale"] if scale is None else scale,
                   num_splits=num_splits)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7, 16])
@pytest.mark.parametrize("L", [1, 40, 64, 300, 1000])
def test_small_decode_with_poisoned_tail(L, splits):
    cfg = DecodeConfig("d", 21, 3, 4, L, 128, "bf16", "scaled", "uniform_half")
    x = decode_inputs(cfg, seed=L, poison=True)
    _say("decode small", L, splits, x["seqlens"].tolist())
    o = _run(x, splits)
    k = torch.nan_to_num(x["k_cache"].float())  # oracle never reads rows >= seqlens
    v = torch.nan_to_num(x["v_cache"].float())
    ref = oracle.decode(x["q"], x["rho"], k, v, x["seqlens"], x["scale"], form="cov")
    check_bf16(o, ref, f"L={L} splits={splits}")


def test_seqlens_edge_cases():
    cfg = DecodeConfig("d", 22, 5, 2, 200, 128, "bf16", "proj32", "full")
    x = decode_inputs(cfg, seed=1)
    sl = torch.tensor([0, -5, 1, 200, 100000], dtype=torch.int32)
    for splits in (1, 4):
        o = _run(x, splits, seqlens=sl).cpu()
        assert torch.all(o[0] == 0) and torch.all(o[1] == 0)
        assert torch.equal(o[2], x["v_cache"][2, :, 0])  # one key: exactly its value
        ref = oracle.decode(x["q"], x["rho"], x["k_cache"], x["v_cache"], sl, x["scale"])
        check_bf16(o[3:], ref[3:], f"edges splits={splits}")


def test_decode_equals_last_prefill_row():
    from plx_synth.inputs import PrefillConfig, prefill_inputs
    p = prefill_inputs(PrefillConfig("p", 23, 2, 2, 333, 128, "bf16", "scaled"), seed=3)
    pd = {k: p[k].to(DEV) for k in ("q", "k", "v", "rho")}
    pre = plx.prefill(pd["q"], pd["k"], pd["v"], pd["rho"], p["scale"]).cpu()
    sl = torch.full((2,), 333, dtype=torch.int32, device=DEV)
    dec = plx.decode(pd["q"][:, :, -1].contiguous(), pd["rho"][:, :, -1].contiguous(), pd["k"],
                     pd["v"], sl, p["scale"], num_splits=3).cpu()
    ref = oracle.decode(p["q"][:, :, -1], p["rho"][:, :, -1], p["k"], p["v"], sl.cpu(),
                        p["scale"])
    check_bf16(dec, ref, "decode")
    check_bf16(pre[:, :, -1], ref, "prefill last row")


def test_split_counts_deterministic_and_permutation_invariant_batch():
    cfg = DecodeConfig("d", 24, 4, 2, 777, 128, "bf16", "scaled", "uniform_half")
    x = decode_inputs(cfg, seed=5)
    for splits in (1, 5):
        assert torch.equal(_run(x, splits), _run(x, splits))
    o = _run(x, 4).cpu()
    perm = torch.tensor([3, 1, 0, 2])
    xp = {k: (x[k][perm] if k != "scale" else x[k]) for k in x}
    assert torch.equal(_run(xp, 4).cpu(), o[perm])


# Wave-range mode (num_splits < 0: that many waves share the (b, h) ranges laid end to end).
# (B, H, L_max, waves): whole (b, h) per slice (8, 16 and 2 (b, h) per wave); pieces cut across
# 2-3 waves; (b, h) cut into ~40 pieces (several merge batches); more waves than rows (empty
# slices); a single (b, h).
@pytest.mark.parametrize("B,H,L,waves", [(8, 4, 300, 4), (21, 3, 64, 4), (8, 4, 300, 16),
                                         (8, 4, 300, 24), (8, 4, 300, 64), (3, 2, 1000, 256),
                                         (1, 1, 40, 4096), (1, 1, 1000, 8)])
def test_wave_range_decode(B, H, L, waves):
    cfg = DecodeConfig("d", 25, B, H, L, 128, "bf16", "scaled", "uniform_half")
    x = decode_inputs(cfg, seed=B * 7 + L, poison=True)
    _say("wave-range", B, H, L, waves, "ws", plx.decode_workspace_size(B, H, L, 128, -waves))
    o = _run(x, -waves)
    k = torch.nan_to_num(x["k_cache"].float())
    v = torch.nan_to_num(x["v_cache"].float())
    ref = oracle.decode(x["q"], x["rho"], k, v, x["seqlens"], x["scale"], form="cov")
    check_bf16(o, ref, f"wave-range B={B} H={H} L={L} waves={waves}")
    assert torch.equal(o, _run(x, -waves))


@pytest.mark.parametrize("waves", [4, 12, 64])  # 21 (b, h): whole, cut, cut
def test_wave_range_seqlens_edge_cases(waves):
    # rho as in the prefill configs: with the strong decode probe (RMSNorm(W_R x), norm ~11)
    # a 37-row context has outputs near 11, where bf16 output spacing alone is 1/16.
    cfg = DecodeConfig("d", 22, 7, 3, 200, 128, "bf16", "scaled", "full")
    x = decode_inputs(cfg, seed=1)
    sl = torch.tensor([0, -5, 1, 200, 100000, 0, 37], dtype=torch.int32)
    o = _run(x, -waves, seqlens=sl).cpu()
    for b in (0, 1, 5):
        assert torch.all(o[b] == 0)
    assert torch.equal(o[2], x["v_cache"][2, :, 0])  # one key: exactly its value
    ref = oracle.decode(x["q"], x["rho"], x["k_cache"], x["v_cache"], sl, x["scale"])
    check_bf16(o[3:5], ref[3:5], f"edges waves={waves}")
    check_bf16(o[6:], ref[6:], f"edges waves={waves}")
    zero = _run(x, -waves, seqlens=torch.zeros(7, dtype=torch.int32)).cpu()
    assert torch.all(zero == 0)


def test_wave_range_permuted_batch():
    # Permuting the batch moves every slice boundary; each order must match the oracle.
    cfg = DecodeConfig("d", 24, 6, 4, 777, 128, "bf16", "scaled", "uniform_half")
    x = decode_inputs(cfg, seed=9)
    ref = oracle.decode(x["q"], x["rho"], x["k_cache"], x["v_cache"], x["seqlens"], x["scale"])
    check_bf16(_run(x, -16), ref, "wave-range")
    perm = torch.tensor([3, 1, 0, 5, 2, 4])
    xp = {k: (x[k][perm] if k != "scale" else x[k]) for k in x}
    check_bf16(_run(xp, -16), ref[perm.numpy()], "wave-range permuted")


def test_auto_plan_modes():
    # Automatic choice (needs the device's compute-unit count): many short sequences use
    # wave-range mode with whole (b, h) per slice (no workspace); the rest use split mode.
    assert plx.decode_num_splits(2048, 16, 128, 0) < 0
    assert plx.decode_workspace_size(2048, 16, 128, 128, 0) == 0
    assert plx.decode_num_splits(1, 16, 32768, 0) > 0
    assert plx.decode_num_splits(16, 16, 1024, 0) > 0
    assert plx.decode_num_splits(2048, 16, 1024, 0) > 0


@pytest.mark.parametrize("splits", [0, 1, 2, 7, 64, 128])
def test_config_decode_32k(splits):
    cfg = CONFIGS["decode_32k"]
    x = decode_inputs(cfg, seed=0)
    _say("decode_32k splits", splits, "->", plx.decode_num_splits(cfg.B, cfg.H, cfg.L_max, splits))
    o = _run(x, splits)
    ref = oracle.decode(x["q"], x["rho"], x["k_cache"], x["v_cache"], x["seqlens"], x["scale"],
                        form="cov" if splits == 0 else "sweighted")
    _say(check_bf16(o, ref, f"decode_32k splits={splits}"))


@pytest.mark.parametrize("cell", decode_grid_cells(), ids=lambda c: c.name)
def test_decode_grid_cell(cell):
    dev_draw = not host_draw_ok(cell)
    _say("grid cell", cell.name, "device draw" if dev_draw else "host draw")
    x = decode_inputs(cell, seed=0, device=DEV, poison=True, device_draw=dev_draw)
    o = plx.decode(x["q"], x["rho"], x["k_cache"], x["v_cache"], x["seqlens"], x["scale"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(cell.B)
    pick = np.unique(np.concatenate([[0, cell.B - 1], rng.integers(0, cell.B, 6)]))
    for b in pick:
        n = int(x["seqlens"][b])
        k = x["k_cache"][b: b + 1, :, :n].float().cpu()
        v = x["v_cache"][b: b + 1, :, :n].float().cpu()
        ref = oracle.decode(x["q"][b: b + 1].cpu(), x["rho"][b: b + 1].cpu(), k, v,
                            np.array([n], np.int32), x["scale"], form="sweighted")
        check_bf16(o[b: b + 1], ref, f"{cell.name} b={b} n={n}")
    del x
    torch.cuda.empty_cache()
