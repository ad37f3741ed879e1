"""Seeded synthetic workloads for Parallax attention (prefill and decode).

Every tensor is drawn from a counter-keyed stream so that any (batch, head)
slice can be regenerated on its own:

    key = SeedSequence([seed, cfg_id, tensor_id, chunk]),  chunk = b * H + h

Host draws use numpy's PCG64 in float64, rounded to float32 and then, for bf16
workloads, to bfloat16 with round-to-nearest-even (torch's conversion).
Decode caches too large to draw on the host in reasonable time are drawn on
the target device with torch's seeded generator instead (``device_draw``); a
check against the oracle then reads those exact bytes back.

The probe rho is an input here. Its recipes follow the workload descriptions:
  * "proj32": rho = RMSNorm_head(W_R x), x ~ N(0,1) of width 32,
    W_R ~ N(0, 0.05^2) of shape [H*d, 32]; RMSNorm per head over d,
    eps = 1e-6, unit weight, no RoPE, no gate;
  * "scaled": rho = 0.1 * RMSNorm_head(N(0,1));
  * "half_zero_heads": heads h < H/2 have rho = 0, the rest "scaled";
  * "zero": rho = 0 everywhere (plain softmax attention).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np
import torch

# tensor ids inside the key
T_Q, T_K, T_V, T_X, T_WR, T_SEQ, T_RHO, T_DO = 0, 1, 2, 3, 4, 5, 6, 7

RMS_EPS = 1e-6


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    cfg_id: int
    B: int
    H: int
    T: int
    d: int
    dtype: str  # "f32" | "bf16"
    rho: str  # "proj32" | "scaled" | "half_zero_heads" | "zero"

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    cfg_id: int
    B: int
    H: int
    L_max: int
    d: int
    dtype: str
    rho: str  # "proj32" | "scaled" | "zero"
    seqlens: str  # "full" | "uniform_half"  (uniform integer in [L_max/2, L_max])

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


def decode_grid_cells():
    """Decode sweep: batch x context at H=16, d=128, dropping B*ctx > 2^23."""
    cells = []
    for B in (1, 16, 128, 512, 2048):
        for ctx in (128, 1024, 4096, 32768):
            if B * ctx > (1 << 23):
                continue
            cells.append(DecodeConfig(f"decode_grid_b{B}_ctx{ctx}", 4, B, 16, ctx, 128,
                                      "bf16", "scaled", "uniform_half"))
    return cells


CONFIGS: Dict[str, object] = {
    "tiny_f32": PrefillConfig("tiny_f32", 1, 1, 2, 64, 16, "f32", "proj32"),
    "prefill_bf16": PrefillConfig("prefill_bf16", 2, 4, 16, 2048, 128, "bf16", "scaled"),
    "decode_32k": DecodeConfig("decode_32k", 3, 1, 16, 32768, 128, "bf16", "proj32", "full"),
    "prefill_long": PrefillConfig("prefill_long", 5, 1, 32, 32768, 128, "bf16",
                                  "half_zero_heads"),
}
for _c in decode_grid_cells():
    CONFIGS[_c.name] = _c


# ----------------------------------------------------------------------------- draws

def _rng(seed: int, cfg_id: int, tensor_id: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(seed), int(cfg_id), int(tensor_id), int(chunk)])))


def _normal_host(shape, seed, cfg_id, tensor_id, chunk, std=1.0) -> np.ndarray:
    return _rng(seed, cfg_id, tensor_id, chunk).standard_normal(shape) * std


def to_dtype(x64, dtype: str) -> torch.Tensor:
    """float64 -> float32 -> (bf16, RNE). Returns a CPU torch tensor."""
    t = torch.as_tensor(np.ascontiguousarray(x64)).to(torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t


def _rms_norm_lastdim(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + RMS_EPS)


def _per_head(shape_bh_rest, seed, cfg_id, tensor_id, H):
    """Draw a [B, H, *rest] float64 tensor one (b, h) chunk at a time."""
    B = shape_bh_rest[0]
    rest = shape_bh_rest[2:]
    out = np.empty(shape_bh_rest, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = _normal_host(rest, seed, cfg_id, tensor_id, b * H + h)
    return out


def _rho_host(kind: str, B: int, H: int, rows: int, d: int, seed: int, cfg_id: int):
    """Probe rows: float64 [B, H, rows, d]."""
    if kind == "zero":
        return np.zeros((B, H, rows, d))
    if kind in ("scaled", "half_zero_heads"):
        r = 0.1 * _rms_norm_lastdim(_per_head((B, H, rows, d), seed, cfg_id, T_RHO, H))
        if kind == "half_zero_heads":
            r[:, : H // 2] = 0.0
        return r
    if kind == "proj32":
        out = np.empty((B, H, rows, d))
        w_r = _normal_host((H * d, 32), seed, cfg_id, T_WR, 0, std=0.05)
        for b in range(B):
            x = _normal_host((rows, 32), seed, cfg_id, T_X, b)
            proj = (x @ w_r.T).reshape(rows, H, d)  # [rows, H, d]
            out[b] = _rms_norm_lastdim(proj).transpose(1, 0, 2)
        return out
    raise ValueError(kind)


# ----------------------------------------------------------------------------- prefill

def prefill_inputs(cfg: PrefillConfig, seed: int = 0, device: Optional[str] = None):
    """q, k, v, rho as contiguous [B, H, T, d] tensors of cfg.dtype (on ``device``)."""
    shp = (cfg.B, cfg.H, cfg.T, cfg.d)
    out = {}
    for name, tid in (("q", T_Q), ("k", T_K), ("v", T_V)):
        out[name] = to_dtype(_per_head(shp, seed, cfg.cfg_id, tid, cfg.H), cfg.dtype)
    out["rho"] = to_dtype(_rho_host(cfg.rho, cfg.B, cfg.H, cfg.T, cfg.d, seed, cfg.cfg_id),
                          cfg.dtype)
    if device is not None:
        out = {k_: t.to(device) for k_, t in out.items()}
    out["scale"] = cfg.scale
    return out


def prefill_head_inputs(cfg: PrefillConfig, b: int, h: int, seed: int = 0):
    """Slice (b, h) of prefill_inputs(cfg, seed) alone, as [1, 1, T, d] tensors: the same
    keyed streams, so it equals the full draw's slice. Probe recipes drawn per (b, h):
    "scaled", "half_zero_heads" and "zero"."""
    if cfg.rho not in ("scaled", "half_zero_heads", "zero"):
        raise ValueError(f"probe recipe {cfg.rho} is not drawn per head")
    shp = (cfg.T, cfg.d)
    chunk = b * cfg.H + h
    out = {name: to_dtype(_normal_host(shp, seed, cfg.cfg_id, tid, chunk)[None, None], cfg.dtype)
           for name, tid in (("q", T_Q), ("k", T_K), ("v", T_V))}
    zero = cfg.rho == "zero" or (cfg.rho == "half_zero_heads" and h < cfg.H // 2)
    r = np.zeros(shp) if zero else 0.1 * _rms_norm_lastdim(
        _normal_host(shp, seed, cfg.cfg_id, T_RHO, chunk))
    out["rho"] = to_dtype(r[None, None], cfg.dtype)
    out["scale"] = cfg.scale
    return out


def prefill_upstream_grad(cfg: PrefillConfig, seed: int = 0) -> torch.Tensor:
    """The gradient arriving at the prefill output for a backward pass: N(0, 1), [B, H, T, d]."""
    return to_dtype(_per_head((cfg.B, cfg.H, cfg.T, cfg.d), seed, cfg.cfg_id, T_DO, cfg.H),
                    cfg.dtype)


def small_prefill(B, H, T, d, dtype="bf16", rho="scaled", seed=0, cfg_id=100):
    """A prefill workload of any size drawn with the same recipe (tests, sweeps)."""
    return prefill_inputs(PrefillConfig(f"custom_{B}x{H}x{T}x{d}", cfg_id, B, H, T, d,
                                        dtype, rho), seed)


# ----------------------------------------------------------------------------- decode

def draw_seqlens(cfg: DecodeConfig, seed: int = 0) -> np.ndarray:
    if cfg.seqlens == "full":
        return np.full(cfg.B, cfg.L_max, dtype=np.int32)
    if cfg.seqlens == "uniform_half":
        lo = cfg.L_max // 2
        return _rng(seed, cfg.cfg_id, T_SEQ, 0).integers(lo, cfg.L_max, size=cfg.B,
                                                          endpoint=True).astype(np.int32)
    raise ValueError(cfg.seqlens)


def host_draw_ok(cfg: DecodeConfig) -> bool:
    """Caches up to 2^28 elements per tensor are drawn on the host."""
    return cfg.B * cfg.H * cfg.L_max * cfg.d <= (1 << 28)


def _device_cache(cfg: DecodeConfig, seed: int, tensor_id: int, device) -> torch.Tensor:
    """[B, H, L_max, d] drawn on ``device`` with torch's seeded generator, per batch row."""
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = torch.empty((cfg.B, cfg.H, cfg.L_max, cfg.d), dtype=tdt, device=device)
    g = torch.Generator(device=device)
    for b in range(cfg.B):
        s = np.random.SeedSequence([seed, cfg.cfg_id, tensor_id, b]).generate_state(2)
        g.manual_seed(int(s[0]) << 32 | int(s[1]))
        out[b] = torch.randn((cfg.H, cfg.L_max, cfg.d), generator=g, device=device,
                             dtype=torch.float32).to(tdt)
    return out


def decode_inputs(cfg: DecodeConfig, seed: int = 0, device: Optional[str] = None,
                  poison: bool = False, device_draw: Optional[bool] = None):
    """q, rho [B,H,d]; k_cache, v_cache [B,H,L_max,d]; seqlens int32 [B].

    poison=True fills every cache row at or beyond seqlens[b] with NaN, so a
    kernel that reads or weights an invalid row shows it.
    """
    if device_draw is None:
        device_draw = not host_draw_ok(cfg)
    B, H, L, d = cfg.B, cfg.H, cfg.L_max, cfg.d
    out = {}
    out["q"] = to_dtype(_per_head((B, H, d), seed, cfg.cfg_id, T_Q, H), cfg.dtype)
    out["rho"] = to_dtype(_rho_host(cfg.rho, B, H, 1, d, seed, cfg.cfg_id)[:, :, 0], cfg.dtype)
    seqlens = draw_seqlens(cfg, seed)
    out["seqlens"] = torch.from_numpy(seqlens)
    if device_draw:
        if device is None:
            raise ValueError("device_draw needs a device")
        out["k_cache"] = _device_cache(cfg, seed, T_K, device)
        out["v_cache"] = _device_cache(cfg, seed, T_V, device)
    else:
        out["k_cache"] = to_dtype(_per_head((B, H, L, d), seed, cfg.cfg_id, T_K, H), cfg.dtype)
        out["v_cache"] = to_dtype(_per_head((B, H, L, d), seed, cfg.cfg_id, T_V, H), cfg.dtype)
    if device is not None:
        out = {k_: t.to(device) for k_, t in out.items()}
    if poison:
        for b in range(B):
            n = int(seqlens[b])
            if n < L:
                out["k_cache"][b, :, n:] = float("nan")
                out["v_cache"][b, :, n:] = float("nan")
    out["scale"] = cfg.scale
    return out


def small_decode(B, H, L_max, d, dtype="bf16", rho="scaled", seqlens="uniform_half",
                 seed=0, cfg_id=101, poison=False):
    return decode_inputs(DecodeConfig(f"custom_dec_{B}x{H}x{L_max}x{d}", cfg_id, B, H, L_max,
                                      d, dtype, rho, seqlens), seed, poison=poison)


__all__ = ["PrefillConfig", "DecodeConfig", "CONFIGS", "decode_grid_cells", "prefill_inputs",
           "prefill_head_inputs",
           "decode_inputs", "small_prefill", "small_decode", "to_dtype", "draw_seqlens",
           "host_draw_ok", "replace"]
