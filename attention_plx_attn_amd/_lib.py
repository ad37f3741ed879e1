"""ctypes binding of libplx_attn.so: argument marshalling only.

Every step of the forward runs in the HIP kernels behind the C ABI (include/plx_attn.h).
Torch provides device memory and the current stream; nothing here computes attention,
and there is no fallback: if the library is missing or a call fails, an error is raised.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libplx_attn.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "plx_attn.h")

PLX_F32, PLX_BF16 = 0, 1
PLX_PREFILL_SPLIT_WEIGHTS = 1
_STATUS = {0: "PLX_OK", 1: "PLX_ERR_NULL_POINTER", 2: "PLX_ERR_INVALID_SHAPE",
           3: "PLX_ERR_INVALID_ARG", 4: "PLX_ERR_UNSUPPORTED", 5: "PLX_ERR_MISALIGNED",
           6: "PLX_ERR_WORKSPACE_TOO_SMALL", 7: "PLX_ERR_HIP"}

_lib = None


class PlxError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.plx_status_string(code).decode() if _lib is not None else ""
        super().__init__(f"{where}: {_STATUS.get(code, code)} ({msg})")


def load() -> ctypes.CDLL:
    """Load libplx_attn.so; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, vp, f32 = ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
    lib.plx_attn_prefill.argtypes = [ctypes.c_int] + [i32] * 5 + [vp] * 5 + [f32, vp]
    lib.plx_attn_prefill.restype = ctypes.c_int
    lib.plx_attn_prefill_ex.argtypes = ([ctypes.c_int] + [i32] * 5 + [vp] * 5 +
                                        [f32, ctypes.c_uint32, vp])
    lib.plx_attn_prefill_ex.restype = ctypes.c_int
    lib.plx_attn_decode_num_splits.argtypes = [i32] * 4 + [ctypes.POINTER(i32)]
    lib.plx_attn_decode_num_splits.restype = ctypes.c_int
    lib.plx_attn_decode_workspace_size.argtypes = [i32] * 5 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.plx_attn_decode_workspace_size.restype = ctypes.c_int
    lib.plx_attn_decode.argtypes = ([ctypes.c_int] + [i32] * 5 + [vp] * 6 +
                                    [f32, i32, vp, ctypes.c_size_t, vp])
    lib.plx_attn_decode.restype = ctypes.c_int
    lib.plx_attn_decode_noalloc.argtypes = ([ctypes.c_int] + [i32] * 5 + [vp] * 6 +
                                            [f32, i32, vp])
    lib.plx_attn_decode_noalloc.restype = ctypes.c_int
    lib.plx_attn_decode_gqa_plan.argtypes = [i32] * 6 + [ctypes.POINTER(i32),
                                                         ctypes.POINTER(ctypes.c_size_t)]
    lib.plx_attn_decode_gqa_plan.restype = ctypes.c_int
    lib.plx_attn_decode_gqa.argtypes = ([ctypes.c_int] + [i32] * 6 + [vp] * 6 +
                                        [f32, i32, vp, ctypes.c_size_t, vp])
    lib.plx_attn_decode_gqa.restype = ctypes.c_int
    lib.plx_attn_decode_paged.argtypes = ([ctypes.c_int] + [i32] * 7 + [vp] * 7 +
                                          [f32, i32, vp, ctypes.c_size_t, vp])
    lib.plx_attn_decode_paged.restype = ctypes.c_int
    lib.plx_attn_decode_paged_gqa.argtypes = ([ctypes.c_int] + [i32] * 8 + [vp] * 7 +
                                              [f32, i32, vp, ctypes.c_size_t, vp])
    lib.plx_attn_decode_paged_gqa.restype = ctypes.c_int
    lib.plx_attn_probe.argtypes = [ctypes.c_int] + [i32] * 5 + [vp] * 5 + [f32, f32, vp, vp]
    lib.plx_attn_probe.restype = ctypes.c_int
    lib.plx_attn_prefill_fwd.argtypes = [ctypes.c_int] + [i32] * 5 + [vp] * 7 + [f32, vp]
    lib.plx_attn_prefill_fwd.restype = ctypes.c_int
    lib.plx_attn_prefill_bwd_workspace_size.argtypes = [i32] * 3 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.plx_attn_prefill_bwd_workspace_size.restype = ctypes.c_int
    lib.plx_attn_prefill_bwd.argtypes = ([ctypes.c_int] + [i32] * 5 + [vp] * 13 +
                                         [ctypes.c_size_t, f32, vp])
    lib.plx_attn_prefill_bwd.restype = ctypes.c_int
    lib.plx_status_string.argtypes = [ctypes.c_int]
    lib.plx_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions():
    """Names of the functions include/plx_attn.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(plx_\w+)\s*\(", text)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PLX_BF16
    if t.dtype == torch.float32:
        return PLX_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(t: torch.Tensor, name: str, dtype, device, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on the same GPU as q ({t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream_handle(stream: Optional[torch.cuda.Stream], device) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream).value or 0


def _bind(stream: Optional[torch.cuda.Stream], *tensors) -> None:
    """Tensors allocated here (outputs, workspaces) are written by kernels on `stream`. The
    caching allocator tracks a block only on the stream that was current at allocation, so
    when the kernels run on another stream it must also wait for that one before it reuses
    the memory (a freed workspace could otherwise be handed out while the kernels still use
    it)."""
    if stream is None:
        return
    for t in tensors:
        if t is not None and stream != torch.cuda.current_stream(t.device):
            t.record_stream(stream)


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rho: Optional[torch.Tensor],
            scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            stream: Optional[torch.cuda.Stream] = None,
            split_weights: bool = False) -> torch.Tensor:
    """Causal Parallax prefill. q, k, rho [B,H,T,d_qk]; v [B,H,T,d_v] -> o [B,H,T,d_v].

    rho=None means rho = 0 exactly (plain softmax attention, the specialised kernel).
    split_weights=True passes the weights to the value products as hi + lo bf16 terms
    (plx_attn_prefill_ex with PLX_PREFILL_SPLIT_WEIGHTS)."""
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d_qk]")
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    _check(q, "q", None, None)
    _check(k, "k", q.dtype, q.device, (B, H, T, dqk))
    if rho is not None:
        _check(rho, "rho", q.dtype, q.device, (B, H, T, dqk))
    _check(v, "v", q.dtype, q.device, (B, H, T, dv))
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
        _bind(stream, out)
    _check(out, "out", q.dtype, q.device, (B, H, T, dv))
    if scale is None:
        scale = dqk ** -0.5
    args = (_dtype_code(q), B, H, T, dqk, dv, q.data_ptr(), k.data_ptr(), v.data_ptr(),
            0 if rho is None else rho.data_ptr(), out.data_ptr(), float(scale))
    if split_weights:
        rc = lib.plx_attn_prefill_ex(*args, PLX_PREFILL_SPLIT_WEIGHTS,
                                     _stream_handle(stream, q.device))
    else:
        rc = lib.plx_attn_prefill(*args, _stream_handle(stream, q.device))
    if rc != 0:
        raise PlxError(rc, "plx_attn_prefill_ex" if split_weights else "plx_attn_prefill")
    return out


def prefill_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rho: Optional[torch.Tensor],
                scale: Optional[float] = None, stream: Optional[torch.cuda.Stream] = None):
    """Causal prefill that also saves what the backward needs (bf16, d = 128).

    Returns (o, vbar, stats): o as prefill(); vbar [B,H,T,d] = O1 / l (bf16); stats
    [B,H,T,2] float32 = (lse, tbar) per query row."""
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    _check(q, "q", None, None)
    for name, t in (("k", k), ("v", v)) + ((("rho", rho),) if rho is not None else ()):
        _check(t, name, q.dtype, q.device, (B, H, T, d))
    o = torch.empty_like(q)
    vbar = torch.empty_like(q)
    stats = torch.empty((B, H, T, 2), dtype=torch.float32, device=q.device)
    _bind(stream, o, vbar, stats)
    if scale is None:
        scale = d ** -0.5
    rc = lib.plx_attn_prefill_fwd(_dtype_code(q), B, H, T, d, d, q.data_ptr(), k.data_ptr(),
                                  v.data_ptr(), 0 if rho is None else rho.data_ptr(),
                                  o.data_ptr(), vbar.data_ptr(), stats.data_ptr(), float(scale),
                                  _stream_handle(stream, q.device))
    if rc != 0:
        raise PlxError(rc, "plx_attn_prefill_fwd")
    return o, vbar, stats


def prefill_bwd_workspace_size(B: int, H: int, T: int) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    rc = lib.plx_attn_prefill_bwd_workspace_size(B, H, T, ctypes.byref(n))
    if rc != 0:
        raise PlxError(rc, "plx_attn_prefill_bwd_workspace_size")
    return n.value


def prefill_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rho: torch.Tensor,
                o: torch.Tensor, vbar: torch.Tensor, stats: torch.Tensor, d_o: torch.Tensor,
                scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None):
    """Backward of the causal prefill (bf16, d = 128): gradients (dq, dk, dv, drho) of
    sum(d_o * o), given the forward's o, vbar and stats from prefill_fwd()."""
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    _check(q, "q", None, None)
    for name, t in (("k", k), ("v", v), ("rho", rho), ("o", o), ("vbar", vbar), ("d_o", d_o)):
        _check(t, name, q.dtype, q.device, (B, H, T, d))
    _check(stats, "stats", torch.float32, q.device, (B, H, T, 2))
    grads = [torch.empty_like(q) for _ in range(4)]
    _bind(stream, *grads)
    need = prefill_bwd_workspace_size(B, H, T)
    if workspace is None:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
        _bind(stream, workspace)
    _check(workspace, "workspace", None, q.device)
    if scale is None:
        scale = d ** -0.5
    rc = lib.plx_attn_prefill_bwd(_dtype_code(q), B, H, T, d, d, q.data_ptr(), k.data_ptr(),
                                  v.data_ptr(), rho.data_ptr(), o.data_ptr(), vbar.data_ptr(),
                                  stats.data_ptr(), d_o.data_ptr(),
                                  *(g.data_ptr() for g in grads), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), float(scale),
                                  _stream_handle(stream, q.device))
    if rc != 0:
        raise PlxError(rc, "plx_attn_prefill_bwd")
    return tuple(grads)


def decode_num_splits(B: int, H: int, L_max: int, num_splits: int = 0) -> int:
    lib = load()
    s = ctypes.c_int32(0)
    rc = lib.plx_attn_decode_num_splits(B, H, L_max, num_splits, ctypes.byref(s))
    if rc != 0:
        raise PlxError(rc, "plx_attn_decode_num_splits")
    return s.value


def decode_workspace_size(B: int, H: int, L_max: int, d_v: int, num_splits: int = 0) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    rc = lib.plx_attn_decode_workspace_size(B, H, L_max, d_v, num_splits, ctypes.byref(n))
    if rc != 0:
        raise PlxError(rc, "plx_attn_decode_workspace_size")
    return n.value


def decode(q: torch.Tensor, rho: Optional[torch.Tensor], k_cache: torch.Tensor, v_cache: torch.Tensor,
           seqlens: torch.Tensor, scale: Optional[float] = None, num_splits: int = 0,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """One decode step. q, rho [B,H,d]; caches [B,H,L_max,d]; seqlens int32 [B] -> [B,H,d].

    rho=None means rho = 0 exactly (plain softmax attention, the specialised kernels)."""
    lib = load()
    if q.dim() != 3:
        raise ValueError("q must be [B, H, d_qk]")
    B, H, dqk = q.shape
    L_max, dv = v_cache.shape[2], v_cache.shape[3]
    _check(q, "q", None, None)
    if rho is not None:
        _check(rho, "rho", q.dtype, q.device, (B, H, dqk))
    _check(k_cache, "k_cache", q.dtype, q.device, (B, H, L_max, dqk))
    _check(v_cache, "v_cache", q.dtype, q.device, (B, H, L_max, dv))
    _check(seqlens, "seqlens", torch.int32, q.device, (B,))
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
        _bind(stream, out)
    _check(out, "out", q.dtype, q.device, (B, H, dv))
    need = decode_workspace_size(B, H, L_max, dv, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
        _bind(stream, workspace)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _check(workspace, "workspace", None, q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if scale is None:
        scale = dqk ** -0.5
    rho_ptr = 0 if rho is None else rho.data_ptr()
    rc = lib.plx_attn_decode(_dtype_code(q), B, H, L_max, dqk, dv, q.data_ptr(), rho_ptr,
                             k_cache.data_ptr(), v_cache.data_ptr(), seqlens.data_ptr(),
                             out.data_ptr(), float(scale), int(num_splits), ws_ptr, ws_bytes,
                             _stream_handle(stream, q.device))
    if rc != 0:
        raise PlxError(rc, "plx_attn_decode")
    return out


def decode_noalloc(q: torch.Tensor, rho: Optional[torch.Tensor], k_cache: torch.Tensor,
                   v_cache: torch.Tensor, seqlens: torch.Tensor, out: torch.Tensor,
                   scale: Optional[float] = None, num_splits: int = 0,
                   stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """decode() through plx_attn_decode_noalloc: the split records live in the library's
    fixed per-GPU scratch, and the caller passes the output, so the call allocates nothing.
    Calls that overlap on one GPU race on that scratch."""
    lib = load()
    if q.dim() != 3:
        raise ValueError("q must be [B, H, d_qk]")
    B, H, dqk = q.shape
    L_max, dv = v_cache.shape[2], v_cache.shape[3]
    _check(q, "q", None, None)
    if rho is not None:
        _check(rho, "rho", q.dtype, q.device, (B, H, dqk))
    _check(k_cache, "k_cache", q.dtype, q.device, (B, H, L_max, dqk))
    _check(v_cache, "v_cache", q.dtype, q.device, (B, H, L_max, dv))
    _check(seqlens, "seqlens", torch.int32, q.device, (B,))
    _check(out, "out", q.dtype, q.device, (B, H, dv))
    if scale is None:
        scale = dqk ** -0.5
    rc = lib.plx_attn_decode_noalloc(_dtype_code(q), B, H, L_max, dqk, dv, q.data_ptr(),
                                     0 if rho is None else rho.data_ptr(), k_cache.data_ptr(),
                                     v_cache.data_ptr(), seqlens.data_ptr(), out.data_ptr(),
                                     float(scale), int(num_splits),
                                     _stream_handle(stream, q.device))
    if rc != 0:
        raise PlxError(rc, "plx_attn_decode_noalloc")
    return out


def probe(x: torch.Tensor, w_r: torch.Tensor, H: int, gamma: Optional[torch.Tensor] = None,
          gate: Optional[torch.Tensor] = None, positions: Optional[torch.Tensor] = None,
          eps: float = 1e-6, rope_base: float = 0.0, out: Optional[torch.Tensor] = None,
          stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Probe producer: x [B,T,C], w_r [H*d,C] -> rho [B,H,T,d] =
    gate_h * RoPE(gamma * RMSNorm_head(x W_R^T)). gamma [d], gate [H] float32; positions
    int32 [B] (token t of sequence b is at positions[b] + t); rope_base 0 = no rotation."""
    lib = load()
    if x.dim() != 3:
        raise ValueError("x must be [B, T, C]")
    B, T, C = x.shape
    if w_r.dim() != 2 or w_r.shape[1] != C or w_r.shape[0] % H != 0:
        raise ValueError(f"w_r has shape {tuple(w_r.shape)}, expected [H*d, {C}]")
    d = w_r.shape[0] // H
    _check(x, "x", None, None)
    _check(w_r, "w_r", x.dtype, x.device, (H * d, C))
    ptrs = []
    for t, name, shape, dt in ((gamma, "gamma", (d,), torch.float32),
                               (gate, "gate", (H,), torch.float32),
                               (positions, "positions", (B,), torch.int32)):
        if t is not None:
            _check(t, name, dt, x.device, shape)
        ptrs.append(0 if t is None else t.data_ptr())
    if out is None:
        out = torch.empty((B, H, T, d), dtype=x.dtype, device=x.device)
        _bind(stream, out)
    _check(out, "out", x.dtype, x.device, (B, H, T, d))
    rc = lib.plx_attn_probe(_dtype_code(x), B, T, C, H, d, x.data_ptr(), w_r.data_ptr(), *ptrs,
                            float(eps), float(rope_base), out.data_ptr(),
                            _stream_handle(stream, x.device))
    if rc != 0:
        raise PlxError(rc, "plx_attn_probe")
    return out


def decode_gqa_plan(B: int, H_q: int, H_kv: int, L_max: int, d_v: int = 128,
                    num_splits: int = 0) -> tuple:
    """(split count, workspace bytes) of a grouped-query decode call."""
    lib = load()
    sp, nb = ctypes.c_int32(0), ctypes.c_size_t(0)
    rc = lib.plx_attn_decode_gqa_plan(B, H_q, H_kv, L_max, d_v, num_splits, ctypes.byref(sp),
                                      ctypes.byref(nb))
    if rc != 0:
        raise PlxError(rc, "plx_attn_decode_gqa_plan")
    return sp.value, nb.value


def decode_gqa(q: torch.Tensor, rho: Optional[torch.Tensor], k_cache: torch.Tensor,
               v_cache: torch.Tensor, seqlens: torch.Tensor, scale: Optional[float] = None,
               num_splits: int = 0, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None,
               stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Decode with grouped query heads: q, rho [B,H_q,d]; caches [B,H_kv,L_max,d] with
    H_q / H_kv in {1, 2, 4, 8}; query head h reads cache head h // (H_q / H_kv)."""
    lib = load()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, H_q, d], the caches [B, H_kv, L_max, d]")
    B, Hq, dqk = q.shape
    Hkv, L_max, dv = k_cache.shape[1], k_cache.shape[2], v_cache.shape[3]
    _check(q, "q", None, None)
    if rho is not None:
        _check(rho, "rho", q.dtype, q.device, (B, Hq, dqk))
    _check(k_cache, "k_cache", q.dtype, q.device, (B, Hkv, L_max, dqk))
    _check(v_cache, "v_cache", q.dtype, q.device, (B, Hkv, L_max, dv))
    _check(seqlens, "seqlens", torch.int32, q.device, (B,))
    if out is None:
        out = torch.empty((B, Hq, dv), dtype=q.dtype, device=q.device)
        _bind(stream, out)
    _check(out, "out", q.dtype, q.device, (B, Hq, dv))
    _, need = decode_gqa_plan(B, Hq, Hkv, L_max, dv, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
        _bind(stream, workspace)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _check(workspace, "workspace", None, q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if scale is None:
        scale = dqk ** -0.5
    rc = lib.plx_attn_decode_gqa(_dtype_code(q), B, Hq, Hkv, L_max, dqk, dv, q.data_ptr(),
                                 0 if rho is None else rho.data_ptr(), k_cache.data_ptr(),
                                 v_cache.data_ptr(), seqlens.data_ptr(), out.data_ptr(),
                                 float(scale), int(num_splits), ws_ptr, ws_bytes,
                                 _stream_handle(stream, q.device))
    if rc != 0:
        raise PlxError(rc, "plx_attn_decode_gqa")
    return out


def decode_paged(q: torch.Tensor, rho: Optional[torch.Tensor], k_pool: torch.Tensor,
                 v_pool: torch.Tensor, block_table: torch.Tensor, seqlens: torch.Tensor,
                 scale: Optional[float] = None, num_splits: int = 0,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Decode over a paged cache: q, rho [B,H,d]; pools [num_blocks,H,block_size,d];
    block_table int32 [B, max_blocks] (rows i*block_size.. of sequence b live in block
    block_table[b, i]); seqlens int32 [B]."""
    lib = load()
    B, H, dqk = q.shape
    nblk, _, bs, dv = v_pool.shape
    max_blocks = block_table.shape[1]
    _check(q, "q", None, None)
    if rho is not None:
        _check(rho, "rho", q.dtype, q.device, (B, H, dqk))
    _check(k_pool, "k_pool", q.dtype, q.device, (nblk, H, bs, dqk))
    _check(v_pool, "v_pool", q.dtype, q.device, (nblk, H, bs, dv))
    _check(block_table, "block_table", torch.int32, q.device, (B, max_blocks))
    _check(seqlens, "seqlens", torch.int32, q.device, (B,))
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
        _bind(stream, out)
    _check(out, "out", q.dtype, q.device, (B, H, dv))
    _, need = decode_gqa_plan(B, H, H, max_blocks * bs, dv, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
        _bind(stream, workspace)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _check(workspace, "workspace", None, q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if scale is None:
        scale = dqk ** -0.5
    rc = lib.plx_attn_decode_paged(_dtype_code(q), B, H, bs, max_blocks, nblk, dqk, dv,
                                   q.data_ptr(), 0 if rho is None else rho.data_ptr(),
                                   k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
                                   seqlens.data_ptr(), out.data_ptr(), float(scale),
                                   int(num_splits), ws_ptr, ws_bytes,
                                   _stream_handle(stream, q.device))
    if rc != 0:
        raise PlxError(rc, "plx_attn_decode_paged")
    return out


def decode_paged_gqa(q: torch.Tensor, rho: Optional[torch.Tensor], k_pool: torch.Tensor,
                     v_pool: torch.Tensor, block_table: torch.Tensor, seqlens: torch.Tensor,
                     scale: Optional[float] = None, num_splits: int = 0,
                     out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Paged decode with grouped query heads: q, rho [B,H_q,d]; pools
    [num_blocks,H_kv,block_size,d] with H_q / H_kv in {1, 2, 4, 8}; block_table int32
    [B, max_blocks]; seqlens int32 [B]. Query head h reads cache head h // (H_q / H_kv)."""
    lib = load()
    if q.dim() != 3 or k_pool.dim() != 4:
        raise ValueError("q must be [B, H_q, d], the pools [num_blocks, H_kv, block_size, d]")
    B, Hq, dqk = q.shape
    nblk, Hkv, bs, dv = v_pool.shape
    max_blocks = block_table.shape[1]
    _check(q, "q", None, None)
    if rho is not None:
        _check(rho, "rho", q.dtype, q.device, (B, Hq, dqk))
    _check(k_pool, "k_pool", q.dtype, q.device, (nblk, Hkv, bs, dqk))
    _check(v_pool, "v_pool", q.dtype, q.device, (nblk, Hkv, bs, dv))
    _check(block_table, "block_table", torch.int32, q.device, (B, max_blocks))
    _check(seqlens, "seqlens", torch.int32, q.device, (B,))
    if out is None:
        out = torch.empty((B, Hq, dv), dtype=q.dtype, device=q.device)
        _bind(stream, out)
    _check(out, "out", q.dtype, q.device, (B, Hq, dv))
    _, need = decode_gqa_plan(B, Hq, Hkv, max_blocks * bs, dv, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
        _bind(stream, workspace)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _check(workspace, "workspace", None, q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if scale is None:
        scale = dqk ** -0.5
    rc = lib.plx_attn_decode_paged_gqa(_dtype_code(q), B, Hq, Hkv, bs, max_blocks, nblk, dqk,
                                       dv, q.data_ptr(), 0 if rho is None else rho.data_ptr(),
                                       k_pool.data_ptr(), v_pool.data_ptr(),
                                       block_table.data_ptr(), seqlens.data_ptr(),
                                       out.data_ptr(), float(scale), int(num_splits), ws_ptr,
                                       ws_bytes, _stream_handle(stream, q.device))
    if rc != 0:
        raise PlxError(rc, "plx_attn_decode_paged_gqa")
    return out
