#!/usr/bin/env python3
"""Benchmark of the Parallax attention forward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic inputs:
  * causal prefill, bf16 in/out, B=4, H=16, T=2048, d=128 (fp32 accumulation), then
  * one decode step, bf16, B=1, H=16, d=128 over a 32768-row KV cache (split-KV partials
    plus the combine kernel).
Inputs are resident in HBM before the timed region, and untimed steps run for --settle-s
seconds before the --warmup steps, so that the timed region sees the clock the GPU holds
under sustained load rather than its ramp. The decode cache is rotated over
several device copies so that successive steps cannot be served from the 256 MB
last-level cache.

Prints ONE JSON line. `value` is the prefill's algorithmic throughput in TFLOP/s
(8*d FLOPs per visible causal (query, key) pair: Q K^T, R K^T, P V and (P*T) V);
the decode figures (tokens/s, algorithmic HBM GB/s) ride along in the same line.
After the timed steps the line also carries, each with its own algorithmic work and roofline
fraction: the same prefill with split weights (`prefill_split_weights`), the long prefill
B1 H32 T32768 (`prefill_long`) and every decode grid cell that moves at least 100 MB
(`decode_grid`, cold caches, each beside the time a plain streaming-read kernel takes for
the same bytes in the same run).
`roofline` describes the dominant kernel (the prefill): its average launch duration is
timed with HIP events on the stream it runs on around 20 back-to-back launches after the
timed steps (an event pair around every launch adds its own dispatch gap, ~5 us); `traffic` comes from committed rocprofv3 counter summaries and is
null when the kernel source changed since they were taken. `cpu_baseline` times the
fp64 oracle's streaming form on the host cores.

Extra modes:
  --sweep [OUT_MD]        time the long prefill (1x32x32768) and the 18 decode grid cells
                          (H16 d128, B x ctx) instead of the step; one JSON line each
  --compare [OUT_MD]      time Parallax against softmax-only attention (rho = NULL) with the
                          same inputs and with twice the heads (equal matrix FLOPs)
  --compare-grid [OUT_MD] the same decode comparisons (and Parallax at d = 64) on every decode
                          grid cell, with the ratios' minimum and maximum
  --gqa [OUT_MD]          time the grouped-query decode (G = 1, 2, 4, 8 query heads per cache
                          head) on a 1x16x32768 cache
  --paged [OUT_MD]        time the paged-cache decode against the contiguous cache
  --probe-producer [OUT_MD]  time the probe producer (x W_R^T, RMSNorm, RoPE, gate) on the
                          prefill step's tokens at C = 32 and C = 2048
  --backward [OUT_MD]     time the training pair on the prefill workload: the forward with
                          saved statistics and the backward (dq, dk, dv, drho)
Used to produce the committed rocprofv3 summaries:
  --calibrate-copy        also run a reference kernel of known traffic (1 GiB read + 1 GiB
                          written), which scales the counters
  --summarize-counters F W [M]  fold rocprofv3 --pmc CSVs (FETCH_SIZE run F, WRITE_SIZE run W,
                            MFMA run M: SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES
                            GRBM_GUI_ACTIVE) into profiles/prefill_bf16_d128_counters.json
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COUNTERS_JSON = os.path.join(ROOT, "profiles", "prefill_bf16_d128_counters.json")
PREFILL_KERNEL = "prefill_bf16_kernel<128>"


def is_prefill_d128(name: str) -> bool:
    """The d = 128 instances of the prefill kernel, by demangled or mangled name."""
    return "prefill_bf16_kernel" in name and ("<128" in name or "ILi128E" in name)
COPY_BYTES = 1 << 30
PREFILL_SOURCES = ("attention_plx_attn_amd/csrc/prefill_bf16.hip",
                   "attention_plx_attn_amd/csrc/plx_device.hpp")
DECODE_SOURCES = ("attention_plx_attn_amd/csrc/decode_bf16.hip",
                  "attention_plx_attn_amd/csrc/decode_step.hpp")


def code_only(text: str) -> str:
    """C++ source without comments and blank lines (what the counters depend on)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def source_hash(files=PREFILL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()


def prefill_flops(B, H, T, d) -> int:
    return 8 * d * B * H * T * (T + 1) // 2


def decode_bytes(seqlens, H, d) -> int:
    kv = int(sum(int(s) for s in seqlens)) * H * (2 * d) * 2
    return kv + len(seqlens) * H * 3 * d * 2  # + q, rho in and o out


# ------------------------------------------------------------------------------ counters

def _pmc_rows(path_glob, counter):
    out = {}
    for path in glob.glob(path_glob, recursive=True):
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                name = row.get("Kernel_Name", "")
                out.setdefault(name, []).append(float(row["Counter_Value"]))
    return out


def _agent_gpu_info(path_glob):
    """(XCDs, SIMDs) of the GPU agent from rocprofv3's agent_info CSV, if present."""
    for path in glob.glob(path_glob, recursive=True):
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Agent_Type") == "GPU":
                    return int(row["Num_Xcc"]), int(row["Simd_Count"])
    return None


def summarize_counters(fetch_glob, write_glob, mfma_glob=None, out_path=COUNTERS_JSON):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the prefill kernel, calibrated by a
    plain copy of known size run in the same process; with mfma_glob, also the matrix-core
    counters of the same kernel (SQ_INSTS_VALU_MFMA_MOPS_BF16: units of 512 FLOP;
    SQ_VALU_MFMA_BUSY_CYCLES summed over SIMDs; GRBM_GUI_ACTIVE summed over the XCDs)."""
    fetch = _pmc_rows(fetch_glob, "FETCH_SIZE")
    write = _pmc_rows(write_glob, "WRITE_SIZE")

    def pick(d, key):
        vals = [v for k, vs in d.items() if key(k) for v in vs]
        return sum(vals) / len(vals) if vals else None

    is_prefill = is_prefill_d128
    is_ref = lambda k: "neg" in k.lower()  # the --calibrate-copy reference kernel  # noqa: E731
    f_k, w_k = pick(fetch, is_prefill), pick(write, is_prefill)
    f_c, w_c = pick(fetch, is_ref), pick(write, is_ref)
    if None in (f_k, w_k, f_c, w_c):
        raise SystemExit(f"missing counters: prefill {f_k} {w_k} copy {f_c} {w_c}")
    copy_kib = COPY_BYTES / 1024.0
    fetch_scale, write_scale = copy_kib / f_c, copy_kib / w_c
    rec = {
        "kernel": PREFILL_KERNEL,
        "workload": "prefill B4 H16 T2048 d128 bf16 causal",
        "fetch_kib_per_dispatch_raw": f_k,
        "write_kib_per_dispatch_raw": w_k,
        "copy_fetch_kib_raw": f_c,
        "copy_write_kib_raw": w_c,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "hbm_bytes_per_dispatch": (f_k * fetch_scale + w_k * write_scale) * 1024.0,
        "source_sha256": source_hash(),
    }
    # The decode call of the same step (split kernel + combine), scaled the same way.
    is_split = lambda k: "decode_split" in k  # noqa: E731
    is_comb = lambda k: "decode_combine" in k  # noqa: E731
    f_s, w_s = pick(fetch, is_split), pick(write, is_split)
    f_m, w_m = pick(fetch, is_comb), pick(write, is_comb)
    if None not in (f_s, w_s, f_m, w_m):
        rec["decode"] = {
            "workload": "decode B1 H16 L32768 d128 bf16 (split kernel + combine)",
            "hbm_bytes_per_call": (f_s * fetch_scale + w_s * write_scale +
                                   f_m * fetch_scale + w_m * write_scale) * 1024.0,
            "split_hbm_bytes_per_dispatch": (f_s * fetch_scale + w_s * write_scale) * 1024.0,
            "source_sha256": source_hash(DECODE_SOURCES),
        }
    if mfma_glob:
        mops = pick(_pmc_rows(mfma_glob, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), is_prefill)
        busy = pick(_pmc_rows(mfma_glob, "SQ_VALU_MFMA_BUSY_CYCLES"), is_prefill)
        gui = pick(_pmc_rows(mfma_glob, "GRBM_GUI_ACTIVE"), is_prefill)
        info = _agent_gpu_info(os.path.join(os.path.dirname(mfma_glob.split("*")[0]) or ".",
                                            "**", "*agent_info.csv"))
        if None in (mops, busy, gui) or info is None:
            raise SystemExit(f"missing MFMA counters: {mops} {busy} {gui} {info}")
        xcc, simds = info
        rec["mfma_flops_per_dispatch"] = mops * 512.0
        rec["mfma_busy_cycles_per_dispatch"] = busy
        rec["gui_active_cycles_per_dispatch_per_xcd"] = gui / xcc
        rec["simds"] = simds
        rec["mfma_busy_frac_profiled"] = busy / (gui / xcc * simds)
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


def committed_counters():
    """The committed counter record of the prefill kernel, or None once its code changed."""
    try:
        with open(COUNTERS_JSON) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash():
        return None
    return rec


def counter_summary(flops, seconds):
    """Matrix-core counters of the prefill kernel from the committed record: executed MFMA
    FLOPs per launch (they include the masked parts of diagonal tiles) and the MFMA-busy
    fraction, both under the profiler and against this run's own launch time."""
    rec = committed_counters()
    if rec is None or "mfma_flops_per_dispatch" not in rec:
        return None
    per_simd_busy_s = rec["mfma_busy_cycles_per_dispatch"] / rec["simds"] / 2.4e9
    return {"mfma_flops_per_launch": rec["mfma_flops_per_dispatch"],
            "mfma_flops_over_algorithmic": round(rec["mfma_flops_per_dispatch"] / flops, 4),
            "mfma_busy_frac_profiled": round(rec["mfma_busy_frac_profiled"], 4),
            "mfma_busy_frac_at_2p4ghz": round(per_simd_busy_s / seconds, 4)}


def committed_traffic():
    rec = committed_counters()
    return None if rec is None else rec.get("hbm_bytes_per_dispatch")


def committed_decode_traffic():
    """HBM bytes per decode call from the committed counters, or None once the decode code
    changed since they were taken."""
    try:
        with open(COUNTERS_JSON) as fh:
            dec = json.load(fh).get("decode")
    except (OSError, ValueError):
        return None
    if not dec or dec.get("source_sha256") != source_hash(DECODE_SOURCES):
        return None
    return dec.get("hbm_bytes_per_call")


# ------------------------------------------------------------------------------ CPU baseline

def cpu_baseline(px, dx):
    import oracle

    cores = oracle.threads()
    t0 = time.perf_counter()
    oracle.prefill(px["q"], px["k"], px["v"], px["rho"], px["scale"], form="stream", block=64)
    t_pre = time.perf_counter() - t0
    B, H, T, d = px["q"].shape
    t0 = time.perf_counter()
    oracle.decode(dx["q"], dx["rho"], dx["k_cache"], dx["v_cache"], dx["seqlens"], dx["scale"],
                  form="stream", block=64)
    t_dec = time.perf_counter() - t0
    # The long prefill (B1 H32 T32768) takes minutes on the host: one of its heads with a
    # probe (head 16) is timed instead, and its rate stands for the whole workload.
    from plx_synth import CONFIGS, prefill_head_inputs

    lcfg = CONFIGS["prefill_long"]
    hx = prefill_head_inputs(lcfg, 0, lcfg.H // 2, seed=0)
    t0 = time.perf_counter()
    oracle.prefill(hx["q"], hx["k"], hx["v"], hx["rho"], hx["scale"], form="stream", block=64)
    t_long = time.perf_counter() - t0
    long_head_flops = prefill_flops(1, 1, lcfg.T, lcfg.d)
    return {
        "value": prefill_flops(B, H, T, d) / t_pre / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"the full prefill workload B{B} H{H} T{T} d{d} in the oracle's fp64 "
                   f"streaming form ({t_pre:.2f} s); decode B1 H16 L32768 in the same form "
                   f"({t_dec:.2f} s); one head (h = {lcfg.H // 2}, with probe) of the long "
                   f"prefill B1 H{lcfg.H} T{lcfg.T} in the same form ({t_long:.2f} s)"),
        "decode_tokens_per_s": dx["q"].shape[0] / t_dec,
        "prefill_long_head_subset": {
            "heads": 1, "seconds": round(t_long, 3),
            "tflops": round(long_head_flops / t_long / 1e12, 4),
            "whole_workload_seconds_extrapolated": round(t_long * lcfg.B * lcfg.H, 1)},
        "cpu_model": _cpu_model(),
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def streaming_read_gbps(torch, dev, stream) -> float:
    """A measured HBM read rate of this board for reference: torch row sums over 1 GiB of
    fp32 (8192 rows; read once, 32 KB written), median of 10 calls after a short warm-up, HIP
    events on the launch stream. (The fastest torch read on MI355X; a dedicated streaming
    kernel reads somewhat faster.)"""
    x = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(8192, dtype=torch.float32, device=dev)
    for _ in range(5):
        torch.sum(x.view(8192, -1), dim=1, out=sink)
    ts = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.sum(x.view(8192, -1), dim=1, out=sink)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del x
    torch.cuda.empty_cache()
    return x_bytes_gbps(1024 ** 3, sorted(ts)[len(ts) // 2])


def x_bytes_gbps(nbytes: int, ms: float) -> float:
    return nbytes / (ms * 1e-3) / 1e9


# ------------------------------------------------------------------------------ sub-records

def _bench_lib():
    """The benchmark's own streaming-read kernel (attention_plx_attn_amd/bench_csrc)."""
    import ctypes

    path = os.path.join(ROOT, "attention_plx_attn_amd", "libplx_bench.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    lib.plx_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.plx_bench_stream_read.restype = ctypes.c_int
    lib.plx_bench_stream_write.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                           ctypes.c_void_p]
    lib.plx_bench_stream_write.restype = ctypes.c_int
    lib.plx_bench_stream_read_rows.argtypes = ([ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 +
                                               [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p])
    lib.plx_bench_stream_read_rows.restype = ctypes.c_int
    return lib


def back_to_back_us(torch, stream, call, n=20, settle_s=0.3):
    """Average time of n launches issued back to back between two events on `stream` (after
    settle_s seconds of untimed calls): an event pair around every launch would add its own
    dispatch gap (several us) to calls this short."""
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        call()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(3):
        e0.record(stream)
        for _ in range(n):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        best = us if best is None else min(best, us)
    return round(best, 2)


class ColdCaches:
    """Reads 1 GiB before a timed call: evicts the L2s and the 256 MB last-level cache without
    leaving dirty lines whose write-back would be charged to the call."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.flush = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        self.sink = torch.empty(1, dtype=torch.float32, device=dev)

    def __call__(self):
        self.torch.sum(self.flush, dim=0, keepdim=True, out=self.sink)


def timed_calls(torch, stream, call, n, cold=None, settle_s=0.0):
    """Median/p10/p90 of n calls bracketed by HIP events on `stream` (after `settle_s` seconds
    of untimed calls and 3 warm-up calls; `cold` runs before each timed call)."""
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        call()
        torch.cuda.synchronize()
    for _ in range(3):
        call()
    ts = []
    for _ in range(n):
        if cold is not None:
            cold()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return _stats_us(ts)


def stream_floor(torch, blib, stream, a, b, nbytes, cold, n=10):
    """Time of the streaming-read kernel over nbytes (half from each of the device tensors a
    and b), cold caches, best median over five grid sizes: the floor for a call that must
    read that many bytes."""
    half = nbytes // 2 // 16 * 16
    assert half <= a.numel() * a.element_size() and half <= b.numel() * b.element_size()
    sink = torch.zeros(1024, dtype=torch.int32, device=a.device)
    h = ctypes_stream(stream)
    best = None
    for grid in (512, 1024, 2048, 4096, 8192):
        def call(grid=grid):
            rc = blib.plx_bench_stream_read(a.data_ptr(), half, b.data_ptr(), half,
                                            sink.data_ptr(), grid, h)
            if rc != 0:
                raise RuntimeError(f"plx_bench_stream_read: HIP error {rc}")
        st = timed_calls(torch, stream, call, n, cold=cold)
        if best is None or st["median_us"] < best["median_us"]:
            best = dict(st, grid=grid, bytes=2 * half)
    return best


def rows_floor(torch, blib, stream, dx, B, H, L_max, cold, n=10):
    """Time of the streaming-read kernel over exactly the cache rows a decode call reads (rows
    below each sequence's length, in the caches' own [B, H, L_max, d] layout), cold caches,
    best median over five grid sizes."""
    sink = torch.zeros(1024, dtype=torch.int32, device=dx["k_cache"].device)
    h = ctypes_stream(stream)
    best = None
    for grid in (512, 1024, 2048, 4096, 8192):
        def call(grid=grid):
            rc = blib.plx_bench_stream_read_rows(dx["k_cache"].data_ptr(), dx["v_cache"].data_ptr(),
                                                 dx["seqlens"].data_ptr(), B, H, L_max,
                                                 sink.data_ptr(), grid, h)
            if rc != 0:
                raise RuntimeError(f"plx_bench_stream_read_rows: HIP error {rc}")
        st = timed_calls(torch, stream, call, n, cold=cold)
        if best is None or st["median_us"] < best["median_us"]:
            best = dict(st, grid=grid)
    return best


def ctypes_stream(stream) -> int:
    import ctypes
    return ctypes.c_void_p(stream.cuda_stream).value or 0


def prefill_split_record(torch, plx, stream, pd, pcfg, default_us, n=20):
    """The same prefill with split weights (hi + lo bf16 terms, PLX_PREFILL_SPLIT_WEIGHTS)."""
    o = torch.empty_like(pd["q"])
    st = timed_calls(torch, stream, lambda: plx.prefill(pd["q"], pd["k"], pd["v"], pd["rho"],
                                                         pcfg.scale, out=o, split_weights=True),
                     n, settle_s=0.3)
    fl = prefill_flops(pcfg.B, pcfg.H, pcfg.T, pcfg.d)
    tf = fl / (st["median_us"] * 1e-6) / 1e12
    return {"workload": f"prefill B{pcfg.B} H{pcfg.H} T{pcfg.T} d{pcfg.d} bf16, split weights",
            **st, "tflops": round(tf, 1), "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "time_over_default": round(st["median_us"] / default_us, 4)}


def prefill_long_record(torch, plx, dev, stream, n=5):
    """The long prefill B1 H32 T32768 d128, inputs drawn on the device with the recipe's
    distributions (q, k, v ~ N(0,1); rho zero on heads < 16, 0.1 RMSNorm(N(0,1)) on the rest)."""
    from plx_synth import CONFIGS

    cfg = CONFIGS["prefill_long"]
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    shp = (cfg.B, cfg.H, cfg.T, cfg.d)
    d = {k: torch.randn(shp, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
         for k in ("q", "k", "v")}
    r = torch.randn(shp, generator=g, device=dev, dtype=torch.float32)
    r = 0.1 * r * torch.rsqrt(r.pow(2).mean(-1, keepdim=True) + 1e-6)
    r[:, : cfg.H // 2] = 0
    d["rho"] = r.to(torch.bfloat16)
    del r
    o = torch.empty_like(d["q"])
    st = timed_calls(torch, stream,
                     lambda: plx.prefill(d["q"], d["k"], d["v"], d["rho"], cfg.scale, out=o), n,
                     settle_s=0.3)
    fl = prefill_flops(cfg.B, cfg.H, cfg.T, cfg.d)
    tf = fl / (st["median_us"] * 1e-6) / 1e12
    del d, o
    torch.cuda.empty_cache()
    return {"workload": f"prefill B{cfg.B} H{cfg.H} T{cfg.T} d{cfg.d} bf16 causal, half the "
                        "heads rho = 0", **st, "flops": fl, "tflops": round(tf, 1),
            "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "tokens_per_s": round(cfg.B * cfg.T / (st["median_us"] * 1e-6), 0)}


def decode_grid_records(torch, plx, dev, stream, min_bytes=100e6, n=10, only=None):
    """Decode grid cells (H16 d128, B x ctx, seqlens ~ U[ctx/2, ctx]) that move at least
    min_bytes, automatic plan, cold caches; each beside two streaming-read floors measured in
    the same run: the same number of KV bytes read contiguously, and exactly the rows the call
    reads, in place (the ragged lengths leave every (b, h)'s rows past its end unread)."""
    from plx_synth import decode_grid_cells, decode_inputs
    from plx_synth.inputs import draw_seqlens

    blib = _bench_lib()
    cold = ColdCaches(torch, dev)
    recs = []
    for cfg in decode_grid_cells():
        nbytes = decode_bytes(draw_seqlens(cfg, 0).tolist(), cfg.H, cfg.d)
        if nbytes < min_bytes or (only is not None and (cfg.B, cfg.L_max) not in only):
            continue
        dx = decode_inputs(cfg, seed=0, device=str(dev), device_draw=True)
        splits = plx.decode_num_splits(cfg.B, cfg.H, cfg.L_max, 0)
        wsb = plx.decode_workspace_size(cfg.B, cfg.H, cfg.L_max, cfg.d, 0)
        ws = torch.empty(max(wsb // 4, 1), dtype=torch.float32, device=dev)
        od = torch.empty_like(dx["q"])
        st = timed_calls(torch, stream,
                         lambda: plx.decode(dx["q"], dx["rho"], dx["k_cache"], dx["v_cache"],
                                            dx["seqlens"], cfg.scale, out=od, workspace=ws),
                         n, cold=cold)
        kv = nbytes - cfg.B * cfg.H * 3 * cfg.d * 2
        fl = stream_floor(torch, blib, stream, dx["k_cache"], dx["v_cache"], kv, cold)
        fr = rows_floor(torch, blib, stream, dx, cfg.B, cfg.H, cfg.L_max, cold)
        gbps = nbytes / (st["median_us"] * 1e-6) / 1e9
        recs.append({"workload": f"decode B{cfg.B} H{cfg.H} ctx{cfg.L_max} d{cfg.d} bf16",
                     **st, "plan": splits, "bytes": nbytes, "hbm_gbps": round(gbps, 1),
                     "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "tokens_per_s": round(cfg.B / (st["median_us"] * 1e-6), 1),
                     "floor_us": fl["median_us"], "floor_bytes": fl["bytes"],
                     "floor_gbps": round(fl["bytes"] / (fl["median_us"] * 1e-6) / 1e9, 1),
                     "time_over_floor": round(st["median_us"] / fl["median_us"], 4),
                     "rows_floor_us": fr["median_us"],
                     "time_over_rows_floor": round(st["median_us"] / fr["median_us"], 4)})
        print(json.dumps(recs[-1]), file=sys.stderr, flush=True)
        del dx, ws, od
        torch.cuda.empty_cache()
    del cold
    torch.cuda.empty_cache()
    return recs


# ------------------------------------------------------------------------------ sweep

def _stats_us(ms_list):
    xs = sorted(ms_list)
    pick = lambda p: xs[min(len(xs) - 1, int(p * len(xs)))] * 1e3  # noqa: E731
    return {"median_us": round(pick(0.5), 2), "p10_us": round(pick(0.1), 2),
            "p90_us": round(pick(0.9), 2)}


def sweep(out_md):
    """Times the long prefill (1x32x32768) and every decode grid cell (H16 d128).

    Decode cells: before each timed call a 1 GiB buffer is read, which evicts the L2s and the
    256 MB last-level cache, so every call streams its cache from HBM; HIP events bracket the
    decode call only. Prints one JSON line per workload and writes a markdown table."""
    import torch

    import attention_plx_attn_amd as plx
    from plx_synth import CONFIGS, decode_grid_cells, decode_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    lines = []

    # long prefill
    cfg = CONFIGS["prefill_long"]
    # Drawn on the device (seeded) with the recipe's distribution: q, k, v ~ N(0,1); rho zero
    # on the first half of the heads and 0.1 RMSNorm(N(0,1)) on the second half.
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    shp = (cfg.B, cfg.H, cfg.T, cfg.d)
    d = {k: torch.randn(shp, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
         for k in ("q", "k", "v")}
    r = torch.randn(shp, generator=g, device=dev, dtype=torch.float32)
    r = 0.1 * r * torch.rsqrt(r.pow(2).mean(-1, keepdim=True) + 1e-6)
    r[:, : cfg.H // 2] = 0
    d["rho"] = r.to(torch.bfloat16)
    del r
    o = torch.empty_like(d["q"])
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:  # settle the clock
        plx.prefill(d["q"], d["k"], d["v"], d["rho"], cfg.scale, out=o)
        torch.cuda.synchronize()
    times = []
    for _ in range(7):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        plx.prefill(d["q"], d["k"], d["v"], d["rho"], cfg.scale, out=o)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    st = _stats_us(times)
    fl = prefill_flops(cfg.B, cfg.H, cfg.T, cfg.d)
    rec = {"workload": f"prefill B{cfg.B} H{cfg.H} T{cfg.T} d{cfg.d} bf16 causal", **st,
           "tflops": round(fl / (st["median_us"] * 1e-6) / 1e12, 1),
           "mfma_frac": round(fl / (st["median_us"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "tokens_per_s": round(cfg.B * cfg.T / (st["median_us"] * 1e-6), 0)}
    print(json.dumps(rec), flush=True)
    lines.append(rec)
    del d, o
    torch.cuda.empty_cache()

    # decode grid
    # Cold caches before every call: reading 1 GiB evicts the 256 MB last-level cache and the
    # L2s without leaving dirty lines whose write-back would be charged to the decode call.
    flush = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(1, dtype=torch.float32, device=dev)
    for cfg in decode_grid_cells():
        dx = decode_inputs(cfg, seed=0, device=str(dev), device_draw=True)
        splits = plx.decode_num_splits(cfg.B, cfg.H, cfg.L_max, 0)
        wsb = plx.decode_workspace_size(cfg.B, cfg.H, cfg.L_max, cfg.d, 0)
        ws = torch.empty(max(wsb // 4, 1), dtype=torch.float32, device=dev)
        od = torch.empty_like(dx["q"])

        def call():
            plx.decode(dx["q"], dx["rho"], dx["k_cache"], dx["v_cache"], dx["seqlens"],
                       cfg.scale, out=od, workspace=ws)

        for _ in range(3):
            call()
        times = []
        iters = 20
        for _ in range(iters):
            torch.sum(flush, dim=0, keepdim=True, out=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        st = _stats_us(times)
        nbytes = decode_bytes(dx["seqlens"].cpu().tolist(), cfg.H, cfg.d)
        gbps = nbytes / (st["median_us"] * 1e-6) / 1e9
        rec = {"workload": f"decode B{cfg.B} H{cfg.H} ctx{cfg.L_max} d{cfg.d} bf16", **st,
               "splits": splits, "bytes": nbytes, "hbm_gbps": round(gbps, 1),
               "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
               "tokens_per_s": round(cfg.B / (st["median_us"] * 1e-6), 1)}
        print(json.dumps(rec), flush=True)
        lines.append(rec)
        del dx, ws, od
        torch.cuda.empty_cache()

    if out_md:
        with open(out_md, "w") as fh:
            fh.write("| workload | median us | p10 us | p90 us | rate | roofline fraction |\n")
            fh.write("|---|---|---|---|---|---|\n")
            for r in lines:
                if "tflops" in r:
                    rate = f"{r['tflops']} TFLOP/s, {r['tokens_per_s']:.3g} tokens/s"
                    frac = f"{100 * r['mfma_frac']:.1f}% of 2.5 PFLOP/s"
                else:
                    plan = (f"{r['splits']} splits" if r["splits"] > 0
                            else f"{-r['splits']} waves, whole (b, h) slices")
                    rate = f"{r['hbm_gbps']} GB/s, {r['tokens_per_s']:,.0f} tokens/s, {plan}"
                    frac = f"{100 * r['hbm_frac']:.1f}% of 8 TB/s"
                fh.write(f"| {r['workload']} | {r['median_us']} | {r['p10_us']} | {r['p90_us']} "
                         f"| {rate} | {frac} |\n")
    return 0


def compare(out_md):
    """The softmax-only comparisons: Parallax against plain softmax attention (rho = NULL, the
    specialised kernels) on the same q, k, v and cache (I/O-matched), and against softmax
    attention with twice the heads, which does the same matrix FLOPs as Parallax
    (compute-matched: Parallax's two score products and two value products per pair). Prefill
    4x16x2048 and decode 1x16x32768, bf16, d = 128; HIP events, median of 20 calls (prefill
    after 0.5 s of untimed calls; decode with a 1 GiB read before each call)."""
    import torch

    import attention_plx_attn_amd as plx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    flush = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(1, dtype=torch.float32, device=dev)

    def bf(shape, s=1.0):
        return (s * torch.randn(shape, generator=g, device=dev)).to(torch.bfloat16)

    def timed(call, cold, n=20):
        if not cold:
            t_end = time.perf_counter() + 0.5
            while time.perf_counter() < t_end:
                call()
                torch.cuda.synchronize()
        for _ in range(3):
            call()
        ts = []
        for _ in range(n):
            if cold:
                torch.sum(flush, dim=0, keepdim=True, out=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return _stats_us(ts)["median_us"]

    rows = []
    B, T, d = 4, 2048, 128
    for name, H, dh, probe in (
            ("Parallax", 16, d, True), ("softmax only, I/O-matched", 16, d, False),
            ("softmax only, compute-matched (2x heads)", 32, d, False),
            ("Parallax, compute-matched (head dim halved, same FLOPs as softmax at d 128)",
             16, d // 2, True)):
        q, k, v = bf((B, H, T, dh)), bf((B, H, T, dh)), bf((B, H, T, dh))
        rho = bf((B, H, T, dh), 0.1) if probe else None
        o = torch.empty_like(q)
        us = timed(lambda: plx.prefill(q, k, v, rho, dh ** -0.5, out=o), cold=False)
        fl = (8 if probe else 4) * dh * B * H * T * (T + 1) // 2
        rows.append({"kernel": "prefill", "variant": name, "shape": f"{B}x{H}x{T} d{dh}",
                     "median_us": us, "tflops": round(fl / us / 1e6, 1)})
        print(json.dumps(rows[-1]), flush=True)
        del q, k, v, rho, o
    L = 32768
    for name, H, dh, probe in (
            ("Parallax", 16, d, True), ("softmax only, I/O-matched", 16, d, False),
            ("softmax only, compute-matched (2x heads)", 32, d, False),
            ("Parallax, compute-matched (head dim halved: half the cache bytes)", 16, d // 2,
             True)):
        q, kc, vc = bf((1, H, dh)), bf((1, H, L, dh)), bf((1, H, L, dh))
        rho = bf((1, H, dh)) if probe else None
        sl = torch.full((1,), L, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        ws = torch.empty(max(plx.decode_workspace_size(1, H, L, dh) // 4, 1),
                         dtype=torch.float32, device=dev)
        us = timed(lambda: plx.decode(q, rho, kc, vc, sl, dh ** -0.5, out=o, workspace=ws),
                   cold=True)
        nbytes = decode_bytes([L], H, dh) - (0 if probe else H * dh * 2)
        rows.append({"kernel": "decode", "variant": name, "shape": f"1x{H}x{L} d{dh}",
                     "median_us": us, "hbm_gbps": round(nbytes / us / 1e3, 1)})
        print(json.dumps(rows[-1]), flush=True)
        del q, kc, vc, rho, o, ws
        torch.cuda.empty_cache()
    if out_md:
        base = {r["kernel"]: r["median_us"] for r in rows if r["variant"] == "Parallax"}
        with open(out_md, "w") as fh:
            fh.write("| kernel | variant | shape | median us | rate | time / Parallax |\n")
            fh.write("|---|---|---|---|---|---|\n")
            for r in rows:
                rate = (f"{r['tflops']} TFLOP/s" if "tflops" in r else f"{r['hbm_gbps']} GB/s")
                fh.write(f"| {r['kernel']} | {r['variant']} | {r['shape']} | {r['median_us']} | "
                         f"{rate} | {r['median_us'] / base[r['kernel']]:.3f} |\n")
    return 0


def compare_grid(out_md):
    """The pages' decode comparison over their sweep (batch x context, the 18 grid cells, H16
    d128, seqlens ~ U[ctx/2, ctx]) with our own kernels standing in for softmax attention:
    Parallax against softmax only (rho = NULL) on the same cache (I/O-matched), against
    softmax only with twice the heads (compute-matched: the same matrix FLOPs, twice the
    cache), and Parallax at head dim 64 (the pages' compute-matched control: the FLOPs of
    softmax attention at d 128, half its cache). Cold caches, HIP events, median of 10, the
    automatic plan of each call. Ratios > 1 mean Parallax is faster."""
    import torch

    import attention_plx_attn_amd as plx
    from plx_synth import decode_grid_cells
    from plx_synth.inputs import draw_seqlens

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    cold = ColdCaches(torch, dev)
    g = torch.Generator(device=dev)
    rows = []

    def bf(shape, s=1.0):
        return (s * torch.randn(shape, generator=g, device=dev)).to(torch.bfloat16)

    def cache(B, H, L, d):
        # per batch row, so that no float32 temporary of the whole cache is needed
        out = torch.empty((B, H, L, d), dtype=torch.bfloat16, device=dev)
        for b in range(B):
            out[b] = torch.randn((H, L, d), generator=g, device=dev).to(torch.bfloat16)
        return out

    def timed(B, H, L, d, probe, sl):
        q = bf((B, H, d))
        rho = bf((B, H, d), 0.1) if probe else None
        kc, vc = cache(B, H, L, d), cache(B, H, L, d)
        o = torch.empty_like(q)
        wsb = plx.decode_workspace_size(B, H, L, d, 0)
        ws = torch.empty(max(wsb // 4, 1), dtype=torch.float32, device=dev)
        st = timed_calls(torch, stream, lambda: plx.decode(q, rho, kc, vc, sl, d ** -0.5, out=o,
                                                           workspace=ws), 10, cold=cold)
        del q, rho, kc, vc, o, ws
        torch.cuda.empty_cache()
        return st["median_us"]

    for cfg in decode_grid_cells():
        g.manual_seed(cfg.B * 100003 + cfg.L_max)
        sl = torch.from_numpy(draw_seqlens(cfg, 0)).to(dev)
        B, H, L = cfg.B, cfg.H, cfg.L_max
        t_plx = timed(B, H, L, 128, True, sl)
        t_io = timed(B, H, L, 128, False, sl)
        t_cm = timed(B, 2 * H, L, 128, False, sl)
        t_64 = timed(B, H, L, 64, True, sl)
        nbytes = decode_bytes(draw_seqlens(cfg, 0).tolist(), H, 128)
        rows.append({"cell": f"B{B} ctx{L}", "bytes": nbytes, "parallax_us": t_plx,
                     "softmax_io_us": t_io, "softmax_2h_us": t_cm, "parallax_d64_us": t_64,
                     "io_ratio": round(t_io / t_plx, 3), "compute_ratio": round(t_cm / t_plx, 3),
                     "d64_vs_softmax_d128": round(t_io / t_64, 3)})
        print(json.dumps(rows[-1]), flush=True)
    if out_md:
        keys = ("io_ratio", "compute_ratio", "d64_vs_softmax_d128")
        with open(out_md, "w") as fh:
            fh.write("| cell (H16) | bytes | Parallax d128 us | softmax only, same cache us | "
                     "softmax only, 2x heads us | Parallax d64 us | I/O-matched ratio | "
                     "compute-matched ratio (2x heads) | compute-matched ratio (d64) |\n")
            fh.write("|---|---|---|---|---|---|---|---|---|\n")
            for r in rows:
                fh.write(f"| {r['cell']} | {r['bytes'] / 1e6:.1f} MB | {r['parallax_us']} | "
                         f"{r['softmax_io_us']} | {r['softmax_2h_us']} | {r['parallax_d64_us']} | "
                         f"{r['io_ratio']} | {r['compute_ratio']} | {r['d64_vs_softmax_d128']} |\n")
            for lab, sel in (("all 18 cells", rows),
                             ("cells of 100 MB or more", [r for r in rows if r["bytes"] >= 1e8])):
                fh.write(f"| min over {lab} | | | | | | " + " | ".join(
                    str(min(r[k] for r in sel)) for k in keys) + " |\n")
                fh.write(f"| max over {lab} | | | | | | " + " | ".join(
                    str(max(r[k] for r in sel)) for k in keys) + " |\n")
    return 0


def gqa(out_md):
    """Decode with grouped query heads at a fixed cache (B=1, H_kv=16, 32768 rows, d=128, then
    d=64): G = 1, 2, 4, 8 query heads per cache head, against the multi-head decode of the
    same cache (G = 1); then short contexts (B=2048, H_kv=8, 64-128 rows each) at G = 1, 4, 8.
    Cold caches (a 1 GiB read before each call), HIP events, median of 20."""
    import torch

    import attention_plx_attn_amd as plx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(17)
    flush = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(8192, dtype=torch.float32, device=dev)

    def timed(call):
        for _ in range(3):
            call()
        ts = []
        for _ in range(20):
            torch.sum(flush.view(8192, -1), dim=1, out=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return _stats_us(ts)["median_us"]

    rows = []
    B, Hkv, L = 1, 16, 32768
    for d in (128, 64):
        kc = torch.randn((B, Hkv, L, d), generator=g, device=dev).to(torch.bfloat16)
        vc = torch.randn((B, Hkv, L, d), generator=g, device=dev).to(torch.bfloat16)
        sl = torch.full((B,), L, dtype=torch.int32, device=dev)
        q16 = torch.randn((B, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
        r16 = (0.1 * torch.randn((B, Hkv, d), generator=g, device=dev)).to(torch.bfloat16)
        o16 = torch.empty_like(q16)
        us = timed(lambda: plx.decode(q16, r16, kc, vc, sl, d ** -0.5, out=o16))
        rows.append({"kernel": "multi-head decode (VALU value products)", "d": d, "G": 1,
                     "H_q": Hkv, "median_us": us})
        for G in (1, 2, 4, 8):
            Hq = Hkv * G
            q = torch.randn((B, Hq, d), generator=g, device=dev).to(torch.bfloat16)
            r = (0.1 * torch.randn((B, Hq, d), generator=g, device=dev)).to(torch.bfloat16)
            o = torch.empty_like(q)
            _, need = plx.decode_gqa_plan(B, Hq, Hkv, L, d)
            ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
            us = timed(lambda: plx.decode_gqa(q, r, kc, vc, sl, d ** -0.5, out=o,
                                              workspace=ws))
            rows.append({"kernel": "grouped-query decode (MFMA value products)", "d": d,
                         "G": G, "H_q": Hq, "median_us": us})
        del kc, vc
        torch.cuda.empty_cache()
    for r_ in rows:
        r_["bytes"] = B * Hkv * L * 2 * r_["d"] * 2 + B * r_["H_q"] * 3 * r_["d"] * 2
    # Short contexts: many sequences of 64-128 rows (chunks of one step per wave, the
    # one-register-set instances), B = 2048, H_kv = 8.
    Bs, Hs, Ls = 2048, 8, 128
    sls = torch.randint(Ls // 2, Ls + 1, (Bs,), generator=g, device=dev, dtype=torch.int32)
    for d in (128, 64):
        kc = torch.randn((Bs, Hs, Ls, d), generator=g, device=dev).to(torch.bfloat16)
        vc = torch.randn((Bs, Hs, Ls, d), generator=g, device=dev).to(torch.bfloat16)
        for G in (1, 4, 8):
            Hq = Hs * G
            q = torch.randn((Bs, Hq, d), generator=g, device=dev).to(torch.bfloat16)
            r = (0.1 * torch.randn((Bs, Hq, d), generator=g, device=dev)).to(torch.bfloat16)
            o = torch.empty_like(q)
            _, need = plx.decode_gqa_plan(Bs, Hq, Hs, Ls, d)
            ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
            us = timed(lambda: plx.decode_gqa(q, r, kc, vc, sls, d ** -0.5, out=o,
                                              workspace=ws))
            rows.append({"kernel": f"grouped-query decode, B{Bs} H_kv{Hs} ctx{Ls} "
                                   f"(seqlens U[{Ls // 2}, {Ls}])", "d": d, "G": G, "H_q": Hq,
                         "B": Bs,
                         "median_us": us,
                         "bytes": int(sls.sum()) * Hs * 2 * d * 2 + Bs * Hq * 3 * d * 2})
        del kc, vc
        torch.cuda.empty_cache()
    for r_ in rows:
        nbytes = r_["bytes"]
        r_["hbm_gbps"] = round(nbytes / r_["median_us"] / 1e3, 1)
        r_["hbm_frac"] = round(r_["hbm_gbps"] / HBM_PEAK_GBPS, 4)
        r_["query_heads_per_s"] = round(r_.get("B", B) * r_["H_q"] / (r_["median_us"] * 1e-6), 0)
        print(json.dumps(r_), flush=True)
    if out_md:
        with open(out_md, "w") as fh:
            fh.write("| kernel | d | G | H_q | median us | HBM GB/s | fraction of 8 TB/s | "
                     "query-head rows / s |\n|---|---|---|---|---|---|---|---|\n")
            for r_ in rows:
                fh.write(f"| {r_['kernel']} | {r_['d']} | {r_['G']} | {r_['H_q']} | "
                         f"{r_['median_us']} | {r_['hbm_gbps']} | {100 * r_['hbm_frac']:.1f}% | "
                         f"{r_['query_heads_per_s']:,.0f} |\n")
    return 0


def paged(out_md):
    """Decode over a paged cache against the contiguous cache, same split plan: B=1, H=16,
    32768 rows and B=16, H=16, 4096 rows (full lengths), and with grouped query heads B=16,
    32 query heads over 8 cache heads, 4096 rows and B=1, 64 over 8, 32768 rows; blocks of 32,
    64 and 256 rows in a random order in the pool, and 64-row blocks in pool order. Cold
    caches (a 1 GiB read before each call), HIP events, median of 20."""
    import torch

    import attention_plx_attn_amd as plx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(19)
    flush = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(8192, dtype=torch.float32, device=dev)

    def timed(call):
        for _ in range(3):
            call()
        ts = []
        for _ in range(20):
            torch.sum(flush.view(8192, -1), dim=1, out=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return _stats_us(ts)["median_us"]

    rows = []
    d = 128
    for B, Hq, H, L in ((1, 16, 16, 32768), (16, 16, 16, 4096), (16, 32, 8, 4096),
                        (1, 64, 8, 32768)):
        grouped = Hq != H
        q = torch.randn((B, Hq, d), generator=g, device=dev).to(torch.bfloat16)
        r = (0.1 * torch.randn((B, Hq, d), generator=g, device=dev)).to(torch.bfloat16)
        kc = torch.randn((B, H, L, d), generator=g, device=dev).to(torch.bfloat16)
        vc = torch.randn((B, H, L, d), generator=g, device=dev).to(torch.bfloat16)
        sl = torch.full((B,), L, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        S, need = plx.decode_gqa_plan(B, Hq, H, L, d)
        ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)
        nbytes = B * H * L * 2 * d * 2 + B * Hq * 3 * d * 2
        name = (f"decode B{B} Hq{Hq} Hkv{H} ctx{L}" if grouped else f"decode B{B} H{H} ctx{L}")
        contiguous = plx.decode_gqa if grouped else plx.decode
        us = timed(lambda: contiguous(q, r, kc, vc, sl, d ** -0.5, num_splits=S, out=o,
                                      workspace=ws))
        rows.append({"workload": name, "cache": "contiguous", "splits": S, "median_us": us})
        paged_call = plx.decode_paged_gqa if grouped else plx.decode_paged
        for bs, shuffled in ((32, True), (64, True), (256, True), (64, False)):
            mb = L // bs
            perm = (torch.randperm(B * mb, generator=torch.Generator().manual_seed(bs))
                    if shuffled else torch.arange(B * mb))
            table = perm.view(B, mb).to(torch.int32).to(dev)
            kp = torch.empty((B * mb, H, bs, d), dtype=torch.bfloat16, device=dev)
            vp = torch.empty_like(kp)
            kp[perm] = kc.view(B, H, mb, bs, d).permute(0, 2, 1, 3, 4).reshape(B * mb, H, bs, d)
            vp[perm] = vc.view(B, H, mb, bs, d).permute(0, 2, 1, 3, 4).reshape(B * mb, H, bs, d)
            us = timed(lambda: paged_call(q, r, kp, vp, table, sl, d ** -0.5, num_splits=S,
                                          out=o, workspace=ws))
            order = "shuffled" if shuffled else "in pool order"
            rows.append({"workload": name, "cache": f"paged, {bs}-row blocks, {order}",
                         "splits": S, "median_us": us})
            del kp, vp
        for r_ in rows[-5:]:
            r_["hbm_gbps"] = round(nbytes / r_["median_us"] / 1e3, 1)
            r_["hbm_frac"] = round(r_["hbm_gbps"] / HBM_PEAK_GBPS, 4)
            print(json.dumps(r_), flush=True)
        del q, r, kc, vc, o, ws
        torch.cuda.empty_cache()
    if out_md:
        with open(out_md, "w") as fh:
            fh.write("| workload | cache | splits | median us | HBM GB/s | fraction of 8 TB/s |\n"
                     "|---|---|---|---|---|---|\n")
            for r_ in rows:
                fh.write(f"| {r_['workload']} | {r_['cache']} | {r_['splits']} | "
                         f"{r_['median_us']} | {r_['hbm_gbps']} | {100 * r_['hbm_frac']:.1f}% |\n")
    return 0


def probe_producer(out_md):
    """Times the probe producer rho = gate * RoPE(gamma * RMSNorm_head(x W_R^T)) on the prefill
    step's tokens (4 x 2048, H = 16, d = 128) at the configs' input width C = 32 (bound by
    writing rho) and at C = 2048 (a model-width projection, bound by the matrix cores): 20
    launches back to back between two events (best of three), after 0.3 s of untimed calls.
    Beside it, a plain streaming write of the same output bytes timed the same way: the floor
    of a call that must write rho."""
    import torch

    import attention_plx_attn_amd as plx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    blib = _bench_lib()
    h = ctypes_stream(stream)
    g = torch.Generator(device=dev)
    g.manual_seed(13)
    B, T, H, d = 4, 2048, 16, 128
    rows = []
    for C in (32, 2048):
        x = torch.randn((B, T, C), generator=g, device=dev).to(torch.bfloat16)
        w = (0.05 * torch.randn((H * d, C), generator=g, device=dev)).to(torch.bfloat16)
        gamma = torch.ones(d, device=dev)
        gate = torch.full((H,), 0.5, device=dev)
        rho = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev)
        us = back_to_back_us(torch, stream, lambda: plx.probe(
            x, w, H, gamma=gamma, gate=gate, eps=1e-6, rope_base=10000.0, out=rho))
        out_bytes = B * H * T * d * 2
        floor = None
        for grid in (512, 1024, 2048, 4096):
            f = back_to_back_us(torch, stream, lambda: blib.plx_bench_stream_write(
                rho.data_ptr(), out_bytes, grid, h), settle_s=0.05)
            floor = f if floor is None else min(floor, f)
        nbytes = (B * T * C + H * d * C + B * H * T * d) * 2
        flops = 2 * B * T * C * H * d
        r = {"workload": f"probe producer {B}x{T} tokens, C={C}, H={H}, d={d}, RoPE + gate",
             "us": us, "gbps": round(nbytes / us / 1e3, 1),
             "tflops": round(flops / us / 1e6, 2),
             "bound": "hbm" if flops / nbytes < 312 else "mfma",
             "write_floor_us": floor, "time_over_write_floor": round(us / floor, 3)}
        r["frac"] = round(r["gbps"] / HBM_PEAK_GBPS if r["bound"] == "hbm"
                          else r["tflops"] / BF16_PEAK_TFLOPS, 4)
        rows.append(r)
        print(json.dumps(r), flush=True)
        del x, w, rho
    if out_md:
        with open(out_md, "w") as fh:
            fh.write("| workload | us per call | HBM GB/s | TFLOP/s | bound | roofline fraction | "
                     "streaming write of rho's bytes, us | call / write |\n")
            fh.write("|---|---|---|---|---|---|---|---|\n")
            for r in rows:
                peak = "8 TB/s" if r["bound"] == "hbm" else "2.5 PFLOP/s"
                fh.write(f"| {r['workload']} | {r['us']} | {r['gbps']} | {r['tflops']} "
                         f"| {r['bound']} | {100 * r['frac']:.1f}% of {peak} | "
                         f"{r['write_floor_us']} | {r['time_over_write_floor']} |\n")
    return 0


def backward(out_md):
    """Times the prefill forward with saved statistics and the backward on the prefill
    workload (B=4, H=16, T=2048, d=128, bf16, probe 0.1 * RMSNorm(N(0,1)), upstream gradient
    N(0,1)); HIP events on the launch stream, median of 20 calls after 0.5 s of untimed
    calls. Algorithmic FLOPs per visible causal pair: 8 d for the forward (Q K^T, R K^T, P V,
    (P*T) V) and 16 d for the backward (the three pair products Q K^T, R K^T, dO V^T, and the
    five accumulating products for dV, dK (two), dQ and dR)."""
    import torch

    import attention_plx_attn_amd as plx
    from plx_synth import CONFIGS, prefill_inputs, prefill_upstream_grad

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    cfg = CONFIGS["prefill_bf16"]
    x = prefill_inputs(cfg, seed=0, device=dev)
    do = prefill_upstream_grad(cfg, seed=0).to(dev)
    o, vbar, stats = plx.prefill_fwd(x["q"], x["k"], x["v"], x["rho"], cfg.scale)
    ws = torch.empty(plx.prefill_bwd_workspace_size(cfg.B, cfg.H, cfg.T) // 4,
                     dtype=torch.float32, device=dev)
    pairs = cfg.B * cfg.H * cfg.T * (cfg.T + 1) // 2
    # the same workload at head dim 64 (the compute-matched head dim)
    x64 = {n: t[..., : cfg.d // 2].contiguous() for n, t in x.items() if n != "scale"}
    do64 = do[..., : cfg.d // 2].contiguous()
    s64 = (cfg.d // 2) ** -0.5
    o64, vbar64, stats64 = plx.prefill_fwd(x64["q"], x64["k"], x64["v"], x64["rho"], s64)
    calls = {
        "forward (plx_attn_prefill)": (
            lambda: plx.prefill(x["q"], x["k"], x["v"], x["rho"], cfg.scale), 8 * cfg.d * pairs),
        "forward with saved statistics (plx_attn_prefill_fwd)": (
            lambda: plx.prefill_fwd(x["q"], x["k"], x["v"], x["rho"], cfg.scale),
            8 * cfg.d * pairs),
        "backward (plx_attn_prefill_bwd: dq/drho and dk/dv kernels)": (
            lambda: plx.prefill_bwd(x["q"], x["k"], x["v"], x["rho"], o, vbar, stats, do,
                                    cfg.scale, workspace=ws), 16 * cfg.d * pairs),
        "forward with saved statistics, d = 64": (
            lambda: plx.prefill_fwd(x64["q"], x64["k"], x64["v"], x64["rho"], s64),
            8 * (cfg.d // 2) * pairs),
        "backward, d = 64": (
            lambda: plx.prefill_bwd(x64["q"], x64["k"], x64["v"], x64["rho"], o64, vbar64,
                                    stats64, do64, s64, workspace=ws), 16 * (cfg.d // 2) * pairs),
    }
    rows = []
    for name, (call, flops) in calls.items():
        t_end = time.perf_counter() + 0.5
        while time.perf_counter() < t_end:
            call()
            torch.cuda.synchronize()
        ts = []
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        us = _stats_us(ts)["median_us"]
        r = {"workload": f"{name}, B{cfg.B} H{cfg.H} T{cfg.T}", "median_us": us,
             "tflops": round(flops / us / 1e6, 1),
             "frac": round(flops / us / 1e6 / BF16_PEAK_TFLOPS, 4)}
        rows.append(r)
        print(json.dumps(r), flush=True)
    if out_md:
        with open(out_md, "w") as fh:
            fh.write("| call | median us | algorithmic TFLOP/s | fraction of 2.5 PFLOP/s |\n")
            fh.write("|---|---|---|---|\n")
            for r in rows:
                fh.write(f"| {r['workload']} | {r['median_us']} | {r['tflops']} | "
                         f"{100 * r['frac']:.1f}% |\n")
    return 0


# ------------------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="untimed steps run for at least this long before the warm-up steps: "
                         "the GPU clock ramps up over the first tens of milliseconds of "
                         "sustained matrix work, and a timed region inside the ramp "
                         "under-reports the steady rate")
    ap.add_argument("--copies", type=int, default=4, help="decode cache copies to rotate")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-grid", action="store_true",
                    help="leave the decode grid cells out of the line")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step only, without the sub-records (profiling runs: the "
                         "long prefill runs the same kernel instance as the step)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize-counters", nargs="+",
                    metavar="CSV_GLOB", help="FETCH_SIZE run, WRITE_SIZE run[, MFMA run]")
    ap.add_argument("--sweep", metavar="OUT_MD", nargs="?", const="",
                    help="time the long prefill and the decode grid instead of the step")
    ap.add_argument("--paged", metavar="OUT_MD", nargs="?", const="",
                    help="time the paged-cache decode instead of the step")
    ap.add_argument("--gqa", metavar="OUT_MD", nargs="?", const="",
                    help="time the grouped-query decode instead of the step")
    ap.add_argument("--probe-producer", metavar="OUT_MD", nargs="?", const="",
                    help="time the probe producer instead of the step")
    ap.add_argument("--backward", metavar="OUT_MD", nargs="?", const="",
                    help="time the prefill forward with statistics and its backward instead "
                         "of the step")
    ap.add_argument("--compare-grid", metavar="OUT_MD", nargs="?", const="",
                    help="the softmax-only comparisons on every decode grid cell instead of "
                         "the step")
    ap.add_argument("--decode-cells", metavar="BxCTX[,BxCTX...]",
                    help="time only these decode grid cells (automatic plan, cold caches, "
                         "beside their streaming floors; one JSON line each) instead of the "
                         "step, e.g. for a kernel trace")
    ap.add_argument("--compare", metavar="OUT_MD", nargs="?", const="",
                    help="time Parallax against softmax-only attention (I/O- and "
                         "compute-matched) instead of the step")
    args = ap.parse_args()

    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the Parallax forward on one GPU only; runs on more than "
              f"one GPU (--gpus {args.gpus}, WORLD_SIZE {world}) are not supported.",
              file=sys.stderr, flush=True)
        return 2

    if args.sweep is not None:
        return sweep(args.sweep)
    if args.compare is not None:
        return compare(args.compare)
    if args.compare_grid is not None:
        return compare_grid(args.compare_grid)
    if args.probe_producer is not None:
        return probe_producer(args.probe_producer)
    if args.gqa is not None:
        return gqa(args.gqa)
    if args.paged is not None:
        return paged(args.paged)
    if args.backward is not None:
        return backward(args.backward)
    if args.decode_cells:
        import torch

        import attention_plx_attn_amd as plx
        cells = {tuple(int(v) for v in c.split("x")) for c in args.decode_cells.split(",")}
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        decode_grid_records(torch, plx, dev, torch.cuda.current_stream(dev), min_bytes=0,
                            only=cells)
        return 0

    import torch

    import attention_plx_attn_amd as plx
    from plx_synth import CONFIGS, decode_inputs, prefill_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pcfg, dcfg = CONFIGS["prefill_bf16"], CONFIGS["decode_32k"]
    px = prefill_inputs(pcfg, seed=0)
    dx = decode_inputs(dcfg, seed=0)
    pd = {k: px[k].to(dev) for k in ("q", "k", "v", "rho")}
    dd = {k: dx[k].to(dev) for k in ("q", "rho", "seqlens")}
    caches = [(dx["k_cache"].to(dev), dx["v_cache"].to(dev))]
    for _ in range(1, max(1, args.copies)):
        caches.append((caches[0][0].clone(), caches[0][1].clone()))
    o_p = torch.empty_like(pd["q"])
    o_d = torch.empty_like(dd["q"])
    splits = plx.decode_num_splits(dcfg.B, dcfg.H, dcfg.L_max, 0)
    ws_bytes = plx.decode_workspace_size(dcfg.B, dcfg.H, dcfg.L_max, dcfg.d, 0)
    ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run_prefill():
        plx.prefill(pd["q"], pd["k"], pd["v"], pd["rho"], pcfg.scale, out=o_p)

    def run_decode(i):
        kc, vc = caches[i % len(caches)]
        plx.decode(dd["q"], dd["rho"], kc, vc, dd["seqlens"], dcfg.scale, out=o_d, workspace=ws)

    if args.calibrate_copy:
        # Reference for the traffic counters: an elementwise negation of 1 GiB of fp32
        # reads exactly COPY_BYTES and writes COPY_BYTES.
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(20):
            run_prefill()
            run_decode(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        run_prefill()
        run_decode(i)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        run_prefill()
        ev[i][1].record(stream)
        run_decode(i)
        ev[i][2].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    pre_ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    dec_ms = sorted(e[1].elapsed_time(e[2]) for e in ev)
    avg = lambda xs: sum(xs) / len(xs)  # noqa: E731
    pct = lambda xs, p: xs[min(len(xs) - 1, int(p * len(xs)))]  # noqa: E731

    # Average launch duration of each kernel: NB launches back to back between two events on
    # the launch stream (the per-step event pairs above add the events' own dispatch gaps to
    # every launch). The rooflines use these.
    NB = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(NB):
        run_prefill()
    e1.record(stream)
    torch.cuda.synchronize()
    pre_b2b_us = e0.elapsed_time(e1) * 1e3 / NB
    e0.record(stream)
    for i in range(NB):
        run_decode(i)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_b2b_us = e0.elapsed_time(e1) * 1e3 / NB

    flops = prefill_flops(pcfg.B, pcfg.H, pcfg.T, pcfg.d)
    pre_avg_s = avg(pre_ms) / 1e3
    tflops = flops / pre_avg_s / 1e12
    dbytes = decode_bytes(dx["seqlens"].tolist(), dcfg.H, dcfg.d)
    dec_avg_s = avg(dec_ms) / 1e3
    dec_gbps = dbytes / dec_avg_s / 1e9
    tflops_b2b = flops / (pre_b2b_us * 1e-6) / 1e12
    dec_gbps_b2b = dbytes / (dec_b2b_us * 1e-6) / 1e9

    traffic = committed_traffic()
    read_gbps = streaming_read_gbps(torch, dev, stream)
    # Sub-records after the timed steps: the split-weights prefill, the long prefill and the
    # bandwidth-dominated decode grid cells (each beside its streaming-read floor).
    n_copies = len(caches)
    split_rec = long_rec = None
    grid_recs = []
    if not args.step_only:
        split_rec = prefill_split_record(torch, plx, stream, pd, pcfg, avg(pre_ms) * 1e3)
        print(json.dumps(split_rec), file=sys.stderr, flush=True)
        del caches
        torch.cuda.empty_cache()
        long_rec = prefill_long_record(torch, plx, dev, stream)
        print(json.dumps(long_rec), file=sys.stderr, flush=True)
        if not args.no_grid:
            grid_recs = decode_grid_records(torch, plx, dev, stream)
    result = {
        "metric": "decode tokens/s & HBM GB/s frac; prefill TFLOP/s & MFMA util (B,H,T,d=128)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v; probe 0.1*RMSNorm(N(0,1)) for prefill, "
                "RMSNorm(W_R x) for decode)",
        "config": {"workload": "parallax forward: causal prefill B4 H16 T2048 d128 + "
                               "decode B1 H16 L32768 d128",
                   "prefill": {"B": pcfg.B, "H": pcfg.H, "T": pcfg.T, "d": pcfg.d},
                   "decode": {"B": dcfg.B, "H": dcfg.H, "L": dcfg.L_max, "d": dcfg.d,
                              "splits": splits, "cache_copies": n_copies}},
        "prefill": {"us_avg": round(avg(pre_ms) * 1e3, 2),
                    "us_p10": round(pct(pre_ms, 0.1) * 1e3, 2),
                    "us_p90": round(pct(pre_ms, 0.9) * 1e3, 2),
                    "tflops": round(tflops, 2),
                    "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                    "tokens_per_s": round(pcfg.B * pcfg.T / pre_avg_s, 1),
                    "us_back_to_back": round(pre_b2b_us, 2)},
        "decode": {"us_avg": round(avg(dec_ms) * 1e3, 2),
                   "us_p10": round(pct(dec_ms, 0.1) * 1e3, 2),
                   "us_p90": round(pct(dec_ms, 0.9) * 1e3, 2),
                   "tokens_per_s": round(dcfg.B / dec_avg_s, 1),
                   "hbm_gbps": round(dec_gbps, 1),
                   "hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                   "frac_of_torch_rowsum_read": round(dec_gbps / read_gbps, 4),
                   "bytes": dbytes,
                   "us_back_to_back": round(dec_b2b_us, 2)},
        "roofline": {"bound": "mfma", "achieved": round(tflops_b2b, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops_b2b / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel": PREFILL_KERNEL,
                     "work_per_launch": flops, "launch_us": round(pre_b2b_us, 2),
                     "counters": counter_summary(flops, pre_b2b_us * 1e-6)},
        "roofline_decode": {"bound": "hbm", "achieved": round(dec_gbps_b2b, 1),
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(dec_gbps_b2b / HBM_PEAK_GBPS, 4),
                            "traffic": committed_decode_traffic(),
                            "work_per_launch": dbytes, "launch_us": round(dec_b2b_us, 2)},
        "prefill_split_weights": split_rec,
        "prefill_long": None if long_rec is None else dict(long_rec, roofline={
            "bound": "mfma", "achieved": long_rec["tflops"], "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": long_rec["mfma_frac"], "traffic": None,
            "work_per_launch": long_rec["flops"]}),
        "decode_grid": grid_recs,
        "wall_s_timed": round(wall, 3),
        "system": {"gpu": torch.cuda.get_device_name(dev),
                   "arch": getattr(torch.cuda.get_device_properties(dev), "gcnArchName", None),
                   "hip": torch.version.hip,
                   "torch": torch.__version__, "cus": torch.cuda.get_device_properties(dev)
                   .multi_processor_count,
                   "measured_hbm_read_gbps_torch_rowsum": round(read_gbps, 1),
                   "source_sha256": source_hash(PREFILL_SOURCES + DECODE_SOURCES)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(px, dx)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
