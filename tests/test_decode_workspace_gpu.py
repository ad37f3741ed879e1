"""The split decode's workspace and graph replays.

With S > 1 chunks per (b, h) the split kernel writes one partial record per chunk into the
caller's workspace and the combine kernel merges them. The workspace needs no particular
contents: these tests fill it with random bytes, or with records of a call with another split
count, and expect the bits of a call on a zeroed workspace; they also check repeated calls on
one workspace and replays of a recorded graph (new inputs copied into the recorded buffers,
eager calls on the same workspace in between), at d = 128 and d = 64, against the fp64 oracle.
"""
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


def _ws(B, H, L, d, splits, fill):
    n = plx.decode_workspace_size(B, H, L, d, splits)
    assert n % 8 == 0 and n > 0
    if fill == "zero":
        return torch.zeros(n // 4, dtype=torch.float32, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(n)
    raw = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g)
    return raw.view(torch.float32).to(DEV)


def _call(g, x, splits, ws, out=None):
    return plx.decode(g["q"], g["rho"], g["k_cache"], g["v_cache"], g["seqlens"], x["scale"],
                      num_splits=splits, out=out, workspace=ws)


def _oracle(x):
    return oracle.decode(x["q"], x["rho"], x["k_cache"], x["v_cache"], x["seqlens"], x["scale"])


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("splits", [2, 5, 16])
def test_workspace_contents_do_not_matter(d, splits):
    B, H, L = 2, 3, 2000
    x = decode_inputs(DecodeConfig("m", 51, B, H, L, d, "bf16", "scaled", "uniform_half"),
                      seed=splits)
    g = _dev(x)
    _say("merge ws", d, splits, x["seqlens"].tolist())
    o0 = _call(g, x, splits, _ws(B, H, L, d, splits, "zero"))
    o1 = _call(g, x, splits, _ws(B, H, L, d, splits, "random"))
    # records of a call with another split count, at other offsets
    other = 16 if splits != 16 else 3
    big = _ws(B, H, L, d, max(splits, other), "zero")
    _call(g, x, other, big)
    o2 = _call(g, x, splits, big)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(o0, o2)
    check_bf16(o0, _oracle(x), f"merge d={d} S={splits}")


@pytest.mark.parametrize("d", [128, 64])
def test_repeated_calls_on_one_workspace(d):
    B, H, L, S = 3, 2, 1500, 7
    x = decode_inputs(DecodeConfig("m", 52, B, H, L, d, "bf16", "proj32", "uniform_half"),
                      seed=d)
    g = _dev(x)
    ws = _ws(B, H, L, d, S, "random")
    outs = [_call(g, x, S, ws) for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    check_bf16(outs[0], _oracle(x), f"repeat d={d}")


@pytest.mark.parametrize("d", [128, 64])
def test_graph_replays_merge_every_time(d):
    """Every replay of a recorded decode (split kernel + combine) gives the eager bits for the
    inputs in the recorded buffers, also after eager calls on the same workspace."""
    B, H, L, S = 2, 4, 4096, 16
    cfg = DecodeConfig("m", 53, B, H, L, d, "bf16", "scaled", "full")
    xs = [decode_inputs(cfg, seed=s) for s in range(4)]
    g = _dev(xs[0])
    ws = _ws(B, H, L, d, S, "random")
    out = torch.empty(B, H, d, dtype=torch.bfloat16, device=DEV)
    eager = []
    for x in xs:  # the eager results, on a workspace of its own
        gx = _dev(x)
        eager.append(_call(gx, x, S, _ws(B, H, L, d, S, "zero")).clone())
    _call(g, xs[0], S, ws, out=out)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _call(g, xs[0], S, ws, out=out)
    torch.cuda.synchronize()
    for rep in range(6):
        x = xs[rep % 4]
        for k in ("q", "rho"):  # new queries into the recorded input buffers
            g[k].copy_(x[k].to(DEV))
        g["k_cache"].copy_(x["k_cache"].to(DEV))
        g["v_cache"].copy_(x["v_cache"].to(DEV))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _say("replay", d, rep)
        assert torch.equal(out, eager[rep % 4]), f"replay {rep}"
        if rep % 2 == 1:  # an eager call on the same workspace between replays
            _call(g, x, S, ws)
            torch.cuda.synchronize()
    check_bf16(eager[0], _oracle(xs[0]), f"graph d={d}")


def test_side_stream_with_internal_workspace():
    """Calls on a side stream whose output and workspace the binding allocates, while the
    current stream allocates and overwrites memory of the same sizes right after each call:
    every result has the bits of a call on the current stream, and matches the oracle."""
    B, H, L, splits = 1, 16, 8192, 16
    x = decode_inputs(DecodeConfig("m", 53, B, H, L, 128, "bf16", "proj32", "full"), seed=0)
    g = _dev(x)
    want = _call(g, x, splits, None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    n_ws = plx.decode_workspace_size(B, H, L, 128, splits) // 4
    outs = []
    for _ in range(8):
        outs.append(plx.decode(g["q"], g["rho"], g["k_cache"], g["v_cache"], g["seqlens"],
                               x["scale"], num_splits=splits, stream=side))
        junk = torch.full((n_ws,), float("nan"), device=DEV)
        junk_o = torch.full((B, H, 128), 7.0, dtype=torch.bfloat16, device=DEV)
        del junk, junk_o
    side.synchronize()
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, want)
    _say("side stream", check_bf16(outs[0], _oracle(x), "side stream"))
