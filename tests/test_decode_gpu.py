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


# rho recipes: "scaled" (0.1 RMSNorm, as the prefill workloads) and "proj32" (the single-step
# decode workload's unit-RMS probe RMSNorm(W_R x): |t| ~ 11, a strong correction).
@pytest.mark.parametrize("rho", ["scaled", "proj32"])
@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7, 16])
@pytest.mark.parametrize("L", [1, 40, 64, 300, 1000])
def test_small_decode_with_poisoned_tail(L, splits, rho):
    cfg = DecodeConfig("d", 21, 3, 4, L, 128, "bf16", rho, "uniform_half")
    x = decode_inputs(cfg, seed=L, poison=True)
    _say("decode small", L, splits, rho, x["seqlens"].tolist())
    o = _run(x, splits)
    k = torch.nan_to_num(x["k_cache"].float())  # oracle never reads rows >= seqlens
    v = torch.nan_to_num(x["v_cache"].float())
    ref = oracle.decode(x["q"], x["rho"], k, v, x["seqlens"], x["scale"], form="cov")
    check_bf16(o, ref, f"L={L} splits={splits} rho={rho}")


@pytest.mark.parametrize("probe", [True, False])
@pytest.mark.parametrize("d", [128, 64])
def test_one_register_set_instance_matches_two_set_bitwise(d, probe):
    """Sequences of at most 128 rows, one chunk each: with a cache of L_max = 128 every wave has
    at most one 32-row step and the one-register-set instance runs; the same rows in a cache of
    L_max = 256 run the two-set (prefetching) instance. Both consume the same steps in the same
    order, so the outputs must be the same bits (and within the bar of the oracle)."""
    cfg = DecodeConfig("d", 24, 6, 4, 256, d, "bf16", "proj32", "full")
    x = decode_inputs(cfg, seed=2)
    sl = torch.tensor([1, 33, 64, 100, 127, 128], dtype=torch.int32)
    q, rho = x["q"].to(DEV), (x["rho"].to(DEV) if probe else None)
    outs = []
    for L in (256, 128):
        kc = x["k_cache"][:, :, :L].contiguous().to(DEV)
        vc = x["v_cache"][:, :, :L].contiguous().to(DEV)
        assert plx.decode_num_splits(6, 4, L, 1) == 1
        outs.append(plx.decode(q, rho, kc, vc, sl.to(DEV), x["scale"], num_splits=1))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    r = x["rho"] if probe else torch.zeros_like(x["rho"])
    ref = oracle.decode(x["q"], r, x["k_cache"], x["v_cache"], sl, x["scale"], form="cov")
    check_bf16(outs[1], ref, f"one-register-set instance d={d} probe={probe}")


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
@pytest.mark.parametrize("rho", ["scaled", "proj32"])
@pytest.mark.parametrize("B,H,L,waves", [(8, 4, 300, 4), (21, 3, 64, 4), (8, 4, 300, 16),
                                         (8, 4, 300, 24), (8, 4, 300, 64), (3, 2, 1000, 256),
                                         (1, 1, 40, 4096), (1, 1, 1000, 8)])
def test_wave_range_decode(B, H, L, waves, rho):
    cfg = DecodeConfig("d", 25, B, H, L, 128, "bf16", rho, "uniform_half")
    x = decode_inputs(cfg, seed=B * 7 + L, poison=True)
    _say("wave-range", B, H, L, waves, rho, "ws",
         plx.decode_workspace_size(B, H, L, 128, -waves))
    o = _run(x, -waves)
    k = torch.nan_to_num(x["k_cache"].float())
    v = torch.nan_to_num(x["v_cache"].float())
    ref = oracle.decode(x["q"], x["rho"], k, v, x["seqlens"], x["scale"], form="cov")
    check_bf16(o, ref, f"wave-range B={B} H={H} L={L} waves={waves} rho={rho}")
    assert torch.equal(o, _run(x, -waves))


@pytest.mark.parametrize("waves", [4, 12, 64])  # 21 (b, h): whole, cut, cut
def test_wave_range_seqlens_edge_cases(waves):
    # The single-step decode workload's probe (RMSNorm(W_R x), norm ~11): a 37-row context has
    # outputs near 11, where the bf16 output spacing is 1/16 (the half-ulp term of the bar).
    cfg = DecodeConfig("d", 22, 7, 3, 200, 128, "bf16", "proj32", "full")
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
    # Automatic choice (needs the device's compute-unit count): split mode everywhere; many
    # short sequences get one chunk per (b, h) (no workspace, the one-step-per-wave kernel).
    assert plx.decode_num_splits(2048, 16, 128, 0) == 1
    assert plx.decode_workspace_size(2048, 16, 128, 128, 0) == 0
    assert plx.decode_num_splits(128, 16, 128, 0) == 1
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


def grid_pick(B: int) -> np.ndarray:
    """Sequences of a grid cell compared with the oracle: all of them up to B = 128, else the
    first, the last and 64 seeded distinct others."""
    if B <= 128:
        return np.arange(B)
    rng = np.random.default_rng(B)
    return np.unique(np.concatenate([[0, B - 1], rng.choice(B, 64, replace=False)]))


@pytest.mark.parametrize("cell", decode_grid_cells(), ids=lambda c: c.name)
def test_decode_grid_cell(cell):
    dev_draw = not host_draw_ok(cell)
    _say("grid cell", cell.name, "device draw" if dev_draw else "host draw")
    x = decode_inputs(cell, seed=0, device=DEV, poison=True, device_draw=dev_draw)
    o = plx.decode(x["q"], x["rho"], x["k_cache"], x["v_cache"], x["seqlens"], x["scale"])
    torch.cuda.synchronize()
    pick = grid_pick(cell.B)
    sl = x["seqlens"].cpu().numpy()
    got, refs = [], []
    for c0 in range(0, len(pick), 8):  # groups of 8 sequences, cut at the group's longest
        idx = pick[c0: c0 + 8]
        n = int(sl[idx].max())
        it = torch.from_numpy(idx).to(DEV)
        k = x["k_cache"][it, :, :n].cpu()
        v = x["v_cache"][it, :, :n].cpu()
        refs.append(oracle.decode(x["q"][it].cpu(), x["rho"][it].cpu(), k, v, sl[idx],
                                  x["scale"], form="sweighted"))
        got.append(o[it].cpu())
        del k, v
    _say(cell.name, len(pick), "sequences",
         check_bf16(torch.cat(got), np.concatenate(refs), f"{cell.name} ({len(pick)} seqs)"))
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d", [128, 64])
def test_decode_at_the_largest_cache(d):
    """The largest cache the ABI accepts for one (b, h): L_max * 256 < 2^31, so 8,388,607 rows
    (2 GiB of keys at d = 128), every row valid, automatic plan. Seven keys spread over the
    range, the last ones at its end, are scaled copies of q so that their scores (about
    2.5-3.5 sqrt(d)) outweigh the 8.4 million others: the output is then of order one and any
    addressing mistake near the 2 GiB offsets shows. Compared with the oracle over all rows."""
    L = (1 << 31) // 256 - 1
    g = torch.Generator(device=DEV)
    g.manual_seed(100 + d)
    q = torch.randn(1, 1, d, generator=g, device=DEV, dtype=torch.bfloat16)
    rho = torch.randn(1, 1, d, generator=g, device=DEV, dtype=torch.bfloat16)
    kc = torch.randn(1, 1, L, d, generator=g, device=DEV, dtype=torch.bfloat16)
    vc = torch.randn(1, 1, L, d, generator=g, device=DEV, dtype=torch.bfloat16)
    spikes = [0, 1, L // 2, L - 1000, L - 33, L - 2, L - 1]
    for i, j in enumerate(spikes):
        kc[0, 0, j] = (q[0, 0].float() * (2.5 + i / 6)).to(torch.bfloat16)
    sl = torch.tensor([L], dtype=torch.int32, device=DEV)
    scale = d ** -0.5
    _say("largest cache d", d, "rows", L, "plan", plx.decode_num_splits(1, 1, L, 0))
    o = plx.decode(q, rho, kc, vc, sl, scale)
    torch.cuda.synchronize()
    ref = oracle.decode(q, rho, kc, vc, sl, scale, form="sweighted")
    _say(check_bf16(o, ref, f"largest cache d={d}"))
    assert float(np.abs(ref).max()) > 0.3  # the spike rows dominate: a meaningful comparison
