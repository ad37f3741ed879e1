"""fp64 CPU oracle for the Parallax attention forward (TEST INFRASTRUCTURE).

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package. The GPU library never links, loads or calls it,
and the two share no code: the only thing both sides consume is the seeded
input generator in ``plx_synth``.

The arithmetic lives in ``plx_oracle.c`` (plain C, fp64, OpenMP over rows); this
module builds it with gcc and marshals numpy arrays. Three forms are exposed:

* ``"cov"``       -- the definition o = o_SA - Sigma_KV rho with the softmax-weighted
                     KV covariance formed explicitly per query
                     [Resumen Tecnico: Parallax ..., "Mecanismo Central"; agihunt review,
                     method paragraph];
* ``"sweighted"`` -- o = sum_j s_ij v_j with s_ij = p_ij (1 - (t_ij - tbar_i))
                     [paper.rainbus.top summary, method steps 2-4];
* ``"stream"``    -- the block-streaming form with one running max and rescale
                     shared by both branches, optionally split into partial states
                     that are merged [paper.rainbus.top summary, method steps 5-6 and
                     the streaming sentences; agihunt review, hardware paragraph].

Pins for every form are in ``tests/test_oracle_pins.py``. The probe producer
(``probe``: rho = gate * RoPE(RMSNorm(x W_R^T)), plain numpy fp64) is in ``probe.py``; the
backward of the causal prefill (``prefill_backward``, numpy fp64) in ``backward.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "plx_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libplx_oracle.so")
_FORMS = {"cov": 0, "sweighted": 1, "stream": 2}
_lib = None


def build(force: bool = True) -> str:
    """Compile plx_oracle.c with gcc (IEEE fp64: no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        # PLX_ORACLE_LIB points the tests' mutation check at a deliberately broken copy.
        path = os.environ.get("PLX_ORACLE_LIB")
        if path is None:
            path = _LIB_PATH
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
                build(force=True)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.plx_oracle_prefill.argtypes = [ctypes.c_int] * 6 + [dp] * 4 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
            ctypes.c_int64, dp]
        lib.plx_oracle_prefill.restype = ctypes.c_int
        lib.plx_oracle_decode.argtypes = [ctypes.c_int] * 6 + [dp] * 4 + [
            ctypes.POINTER(ctypes.c_int32), ctypes.c_double, ctypes.c_int, ctypes.c_int, dp]
        lib.plx_oracle_decode.restype = ctypes.c_int
        lib.plx_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def prefill(q, k, v, rho, scale: float, form: str = "cov", block: int = 64, splits: int = 1,
            rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Causal Parallax forward for q, k, rho [B,H,T,dqk], v [B,H,T,dv].

    Returns [B,H,T,dv], or [len(rows), dv] for flat row indices (b*H + h)*T + i.
    """
    q, k, v, rho = _f64(q), _f64(k), _f64(v), _f64(rho)
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, T, dqk) and rho.shape == (B, H, T, dqk) and v.shape == (B, H, T, dv)
    lib = _load()
    if rows is None:
        out = np.empty((B, H, T, dv))
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((rows.size, dv))
        rp, nr = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows.size
    rc = lib.plx_oracle_prefill(_FORMS[form], B, H, T, dqk, dv, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(rho), float(scale), int(block), int(splits), rp, nr,
                                _ptr(out))
    if rc != 0:
        raise ValueError("plx_oracle_prefill rejected its arguments")
    return out


def decode(q, rho, k_cache, v_cache, seqlens, scale: float, form: str = "cov", block: int = 64,
           splits: int = 1) -> np.ndarray:
    """One decode step: q, rho [B,H,dqk]; caches [B,H,L_max,d]; seqlens int [B] -> [B,H,dv]."""
    q, rho, k, v = _f64(q), _f64(rho), _f64(k_cache), _f64(v_cache)
    B, H, dqk = q.shape
    L_max, dv = v.shape[2], v.shape[3]
    assert k.shape == (B, H, L_max, dqk) and rho.shape == (B, H, dqk)
    if hasattr(seqlens, "detach"):
        seqlens = seqlens.detach().cpu().numpy()
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    assert sl.shape == (B,)
    out = np.empty((B, H, dv))
    rc = _load().plx_oracle_decode(_FORMS[form], B, H, L_max, dqk, dv, _ptr(q), _ptr(rho),
                                   _ptr(k), _ptr(v),
                                   sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   float(scale), int(block), int(splits), _ptr(out))
    if rc != 0:
        raise ValueError("plx_oracle_decode rejected its arguments")
    return out


def threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().plx_oracle_threads())


from .backward import prefill_backward, prefill_stats  # noqa: E402
from .probe import probe  # noqa: E402

__all__ = ["build", "prefill", "decode", "threads", "probe", "prefill_backward",
           "prefill_stats"]
