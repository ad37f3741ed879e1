"""The C-ABI library loads, exports what include/plx_attn.h declares, and rejects bad
arguments on the host before any HIP call (these tests need no GPU)."""
import ctypes
import subprocess

import pytest

import attention_plx_attn_amd as plx
from attention_plx_attn_amd import _lib

A = 1 << 20  # a 16-byte aligned fake address: validation must reject before using it


@pytest.fixture(scope="module")
def lib():
    return plx.load()


def test_exports_every_declared_symbol(lib):
    declared = plx.header_functions()
    assert set(declared) == {"plx_attn_prefill", "plx_attn_prefill_ex", "plx_attn_decode",
                             "plx_attn_decode_noalloc", "plx_attn_decode_num_splits",
                             "plx_attn_decode_workspace_size", "plx_attn_probe",
                             "plx_attn_decode_gqa", "plx_attn_decode_gqa_plan",
                             "plx_attn_decode_paged", "plx_attn_decode_paged_gqa",
                             "plx_attn_prefill_fwd",
                             "plx_attn_prefill_bwd", "plx_attn_prefill_bwd_workspace_size",
                             "plx_status_string"}
    out = subprocess.run(["nm", "-D", "--defined-only", plx.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for code in range(8):
        s = lib.plx_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.plx_status_string(99) == b"unknown status"


def _prefill(lib, dtype=1, B=1, H=1, T=8, dqk=128, dv=128, ptrs=(A,) * 5, scale=0.1):
    return lib.plx_attn_prefill(dtype, B, H, T, dqk, dv, *ptrs, ctypes.c_float(scale), None)


def test_prefill_validation(lib):
    assert _prefill(lib, ptrs=(0, A, A, A, A)) == 1
    assert _prefill(lib, ptrs=(A, A, A, A, 0)) == 1
    assert _prefill(lib, ptrs=(A, A, A, 0, A), T=0) == 2  # rho may be NULL (softmax only)
    assert _prefill(lib, T=0) == 2
    assert _prefill(lib, B=-1) == 2
    assert _prefill(lib, H=0) == 2
    assert _prefill(lib, T=1 << 24) == 2                 # slice > 2^31 bytes
    assert _prefill(lib, scale=float("nan")) == 3
    assert _prefill(lib, scale=float("inf")) == 3
    assert _prefill(lib, scale=-1.0) == 3
    assert _prefill(lib, dtype=7) == 3
    assert _prefill(lib, dqk=32, dv=32) == 4              # bf16 only at d in {64, 128}
    assert _prefill(lib, dqk=96, dv=96) == 4
    assert _prefill(lib, dqk=128, dv=64) == 4
    assert _prefill(lib, dtype=0, dqk=128, dv=128) == 4   # f32 only at d in {16, 32, 64}
    assert _prefill(lib, dtype=0, dqk=48, dv=48) == 4
    assert _prefill(lib, ptrs=(A + 8, A, A, A, A)) == 5
    assert _prefill(lib, dtype=0, dqk=16, dv=16, ptrs=(A, A, A, A + 4, A)) == 5


def _prefill_ex(lib, flags, dtype=1, T=8, ptrs=(A,) * 5):
    return lib.plx_attn_prefill_ex(dtype, 1, 1, T, 128, 128, *ptrs, ctypes.c_float(0.1), flags,
                                   None)


def test_prefill_ex_validation(lib):
    # the flags word: unknown bits are rejected before anything else is looked at
    assert _prefill_ex(lib, 2) == 3
    assert _prefill_ex(lib, 0x80000000) == 3
    assert _prefill_ex(lib, 1 | 4) == 3
    # the same checks as plx_attn_prefill with a valid flags word
    assert _prefill_ex(lib, 1, ptrs=(0, A, A, A, A)) == 1
    assert _prefill_ex(lib, 1, T=0) == 2
    assert _prefill_ex(lib, 1, dtype=7) == 3
    assert _prefill_ex(lib, 1, ptrs=(A + 8, A, A, A, A)) == 5


def _decode(lib, dtype=1, B=2, H=2, L=64, dqk=128, dv=128, q=A, rho=A, kc=A, vc=A, sl=A, o=A,
            scale=0.1, splits=1, ws=0, wsb=0):
    return lib.plx_attn_decode(dtype, B, H, L, dqk, dv, q, rho, kc, vc, sl, o,
                               ctypes.c_float(scale), splits, ws, wsb, None)


def test_decode_validation(lib):
    assert _decode(lib, sl=0) == 1
    assert _decode(lib, kc=0) == 1
    assert _decode(lib, L=0) == 2
    assert _decode(lib, rho=0, L=0) == 2                  # rho may be NULL (softmax only)
    assert _decode(lib, L=1 << 23) == 2
    assert _decode(lib, B=70000) == 2
    assert _decode(lib, scale=float("nan")) == 3
    assert _decode(lib, splits=-70000) == 3
    assert _decode(lib, B=9000, splits=-8) == 4       # wave-range mode keeps B + 1 sums in LDS
    assert _decode(lib, B=64, H=64, L=1 << 20, splits=-8) == 4  # flat rows must fit in int32
    assert _decode(lib, splits=5000) == 3
    assert _decode(lib, dtype=0) == 4
    assert _decode(lib, dqk=32, dv=32) == 4               # bf16 at d in {64, 128}
    assert _decode(lib, dqk=64, dv=128) == 4
    assert _decode(lib, dqk=64, dv=64, splits=-8) == 4    # wave-range mode: d = 128 only
    assert _decode(lib, vc=A + 2) == 5
    assert _decode(lib, sl=A + 2) == 5
    # split run: the workspace is required and must be large enough
    assert _decode(lib, L=1024, splits=4) == 1
    assert _decode(lib, L=1024, splits=4, ws=A, wsb=100) == 6
    need = 2 * 2 * 4 * (2 * 128 + 4) * 4
    assert _decode(lib, L=1024, splits=4, ws=A + 4, wsb=need) == 5


def test_split_plan_explicit(lib):
    assert plx.decode_num_splits(1, 16, 32768, 32) == 32
    assert plx.decode_num_splits(1, 16, 1000, 3) == 3       # chunks of 384 keys
    assert plx.decode_num_splits(1, 16, 100, 8) == 2        # chunks round up to 64 keys
    assert plx.decode_num_splits(4, 4, 64, 1) == 1
    assert plx.decode_workspace_size(2, 3, 4096, 128, 1) == 0
    assert plx.decode_workspace_size(2, 3, 4096, 128, 4) == 2 * 3 * 4 * 260 * 4
    with pytest.raises(_lib.PlxError):
        plx.decode_num_splits(0, 1, 10, 1)


def test_wave_range_plan_explicit(lib):
    # num_splits < 0 asks for wave-range mode with that many waves, rounded up to 4; the plan
    # reports minus the wave count. Slices end at (b, h) starts (no workspace) once there are
    # at least 2 (b, h) per wave, else each wave has two partial slots.
    assert plx.decode_num_splits(8, 4, 300, -4) == -4
    assert plx.decode_num_splits(8, 4, 300, -5) == -8
    assert plx.decode_workspace_size(8, 4, 300, 128, -16) == 0         # 32 (b, h) >= 2 * 16
    assert plx.decode_workspace_size(8, 4, 300, 128, -20) == 20 * 2 * 260 * 4
    assert plx.decode_workspace_size(1, 1, 40, 128, -4096) == 4096 * 2 * 260 * 4


def _probe(lib, dtype=1, B=2, T=3, C=32, H=2, d=128, x=A, w=A, gamma=0, gate=0, pos=0, eps=1e-6,
           base=0.0, rho=A):
    return lib.plx_attn_probe(dtype, B, T, C, H, d, x, w, gamma, gate, pos, ctypes.c_float(eps),
                              ctypes.c_float(base), rho, None)


def test_probe_validation(lib):
    assert _probe(lib, x=0) == 1
    assert _probe(lib, rho=0) == 1
    assert _probe(lib, T=0) == 2
    assert _probe(lib, C=-8) == 2
    assert _probe(lib, B=1 << 16, T=1 << 12, C=64) == 2       # B*T*C*2 >= 2^31
    assert _probe(lib, eps=-1.0) == 3
    assert _probe(lib, eps=float("nan")) == 3
    assert _probe(lib, base=0.5) == 3                         # RoPE base must exceed 1
    assert _probe(lib, dtype=5) == 3
    assert _probe(lib, d=64) == 4
    assert _probe(lib, C=36) == 4                             # C a multiple of 8
    assert _probe(lib, dtype=0) == 4
    assert _probe(lib, x=A + 8) == 5
    assert _probe(lib, gate=A + 2) == 5
    assert _probe(lib, gamma=A + 4) == 5


def _gqa(lib, dtype=1, B=2, Hq=8, Hkv=2, L=64, dqk=128, dv=128, q=A, rho=A, kc=A, vc=A, sl=A,
         o=A, scale=0.1, splits=1, ws=0, wsb=0):
    return lib.plx_attn_decode_gqa(dtype, B, Hq, Hkv, L, dqk, dv, q, rho, kc, vc, sl, o,
                                   ctypes.c_float(scale), splits, ws, wsb, None)


def test_decode_gqa_validation(lib):
    assert _gqa(lib, q=0) == 1
    assert _gqa(lib, rho=0, L=0) == 2                      # rho may be NULL
    assert _gqa(lib, Hkv=3) == 2                           # H_q not a multiple of H_kv
    assert _gqa(lib, Hkv=0) == 2
    assert _gqa(lib, Hq=6, Hkv=2) == 4                     # G = 3 not built
    assert _gqa(lib, Hq=32, Hkv=2) == 4                    # G = 16 > 8
    assert _gqa(lib, splits=-4) == 3                       # split mode only
    assert _gqa(lib, dqk=32, dv=32) == 4
    assert _gqa(lib, dqk=64, dv=128) == 4
    assert _gqa(lib, kc=A + 8) == 5
    assert _gqa(lib, L=1024, splits=4) == 1                # workspace required
    need = 2 * 8 * 4 * (2 * 128 + 4) * 4
    assert _gqa(lib, L=1024, splits=4, ws=A, wsb=need - 4) == 6
    assert plx.decode_gqa_plan(2, 8, 2, 1024, 128, 4) == (4, need)
    assert plx.decode_gqa_plan(2, 8, 2, 1024, 128, 1) == (1, 0)


def _paged(lib, dtype=1, B=2, H=2, bs=64, mb=4, nb=8, dqk=128, dv=128, q=A, rho=A, kp=A, vp=A,
           tab=A, sl=A, o=A, scale=0.1, splits=1, ws=0, wsb=0):
    return lib.plx_attn_decode_paged(dtype, B, H, bs, mb, nb, dqk, dv, q, rho, kp, vp, tab, sl,
                                     o, ctypes.c_float(scale), splits, ws, wsb, None)


def test_decode_paged_validation(lib):
    assert _paged(lib, tab=0) == 1
    assert _paged(lib, rho=0, B=0) == 2                    # rho may be NULL
    assert _paged(lib, bs=48) == 2                         # block size a power of two
    assert _paged(lib, bs=16) == 2                         # at least 32 rows
    assert _paged(lib, mb=0) == 2
    assert _paged(lib, nb=0) == 2
    assert _paged(lib, splits=-1) == 3
    assert _paged(lib, dqk=32, dv=32) == 4
    assert _paged(lib, dqk=64, dv=128) == 4
    assert _paged(lib, tab=A + 2) == 5
    assert _paged(lib, mb=16, splits=4) == 1               # workspace required


def _paged_gqa(lib, dtype=1, B=2, Hq=8, Hkv=2, bs=64, mb=4, nb=8, dqk=128, dv=128, q=A, rho=A,
               kp=A, vp=A, tab=A, sl=A, o=A, scale=0.1, splits=1, ws=0, wsb=0):
    return lib.plx_attn_decode_paged_gqa(dtype, B, Hq, Hkv, bs, mb, nb, dqk, dv, q, rho, kp, vp,
                                         tab, sl, o, ctypes.c_float(scale), splits, ws, wsb,
                                         None)


def test_decode_paged_gqa_validation(lib):
    assert _paged_gqa(lib, kp=0) == 1
    assert _paged_gqa(lib, tab=0) == 1
    assert _paged_gqa(lib, B=0) == 2
    assert _paged_gqa(lib, Hq=6, Hkv=4) == 2               # H_q a multiple of H_kv
    assert _paged_gqa(lib, Hkv=0) == 2
    assert _paged_gqa(lib, bs=96) == 2                     # block size a power of two
    assert _paged_gqa(lib, bs=16) == 2                     # at least 32 rows
    assert _paged_gqa(lib, mb=0) == 2
    assert _paged_gqa(lib, nb=0) == 2
    assert _paged_gqa(lib, splits=-1) == 3
    assert _paged_gqa(lib, scale=float("nan")) == 3
    assert _paged_gqa(lib, dtype=5) == 3
    assert _paged_gqa(lib, Hq=6, Hkv=2) == 4               # G = 3 not built
    assert _paged_gqa(lib, Hq=32, Hkv=2) == 4              # G = 16 not built
    assert _paged_gqa(lib, dqk=32, dv=32) == 4
    assert _paged_gqa(lib, dqk=64, dv=128) == 4
    assert _paged_gqa(lib, dtype=0) == 4                   # fp32 not built
    assert _paged_gqa(lib, vp=A + 8) == 5
    assert _paged_gqa(lib, tab=A + 2) == 5
    assert _paged_gqa(lib, mb=16, splits=4) == 1           # workspace required
    need = 2 * 8 * 4 * (2 * 128 + 4) * 4
    assert _paged_gqa(lib, mb=16, splits=4, ws=A, wsb=need - 4) == 6


def _fwd(lib, dtype=1, B=1, H=2, T=64, dqk=128, dv=128, q=A, k=A, v=A, rho=A, o=A, vbar=A,
         stats=A, scale=0.1):
    return lib.plx_attn_prefill_fwd(dtype, B, H, T, dqk, dv, q, k, v, rho, o, vbar, stats,
                                    scale, None)


def _bwd(lib, dtype=1, B=1, H=2, T=64, dqk=128, dv=128, ptrs=None, ws_bytes=None, scale=0.1):
    p = dict.fromkeys(("q", "k", "v", "rho", "o", "vbar", "stats", "d_o", "dq", "dk", "dv",
                       "drho", "ws"), A)
    p.update(ptrs or {})
    if ws_bytes is None:
        ws_bytes = B * H * T * 16
    return lib.plx_attn_prefill_bwd(dtype, B, H, T, dqk, dv, *p.values(), ws_bytes, scale, None)


def test_prefill_fwd_validation(lib):
    assert _fwd(lib, vbar=0) == 1
    assert _fwd(lib, stats=0) == 1
    assert _fwd(lib, o=0) == 1
    assert _fwd(lib, T=0) == 2
    assert _fwd(lib, T=1 << 23) == 2                          # T * 256 >= 2^31
    assert _fwd(lib, scale=-1.0) == 3
    assert _fwd(lib, dtype=7) == 3
    assert _fwd(lib, dtype=0) == 4                            # fp32 not built
    assert _fwd(lib, dqk=32, dv=32) == 4
    assert _fwd(lib, dqk=64, dv=128) == 4
    assert _fwd(lib, stats=A + 4) == 5
    assert _fwd(lib, vbar=A + 2) == 5


def test_prefill_bwd_validation(lib):
    n = ctypes.c_size_t(0)
    assert lib.plx_attn_prefill_bwd_workspace_size(2, 3, 100, ctypes.byref(n)) == 0
    assert n.value == 2 * 3 * 100 * 16
    assert lib.plx_attn_prefill_bwd_workspace_size(2, 0, 100, ctypes.byref(n)) == 2
    assert lib.plx_attn_prefill_bwd_workspace_size(2, 3, 100, None) == 1
    for name in ("q", "k", "v", "rho", "o", "vbar", "stats", "d_o", "dq", "dk", "dv", "drho",
                 "ws"):
        assert _bwd(lib, ptrs={name: 0}) == 1, name
        assert _bwd(lib, ptrs={name: A + 8}) == 5, name
    assert _bwd(lib, T=-1) == 2
    assert _bwd(lib, scale=float("inf")) == 3
    assert _bwd(lib, dtype=0) == 4
    assert _bwd(lib, dqk=128, dv=64) == 4
    assert _bwd(lib, ws_bytes=1 * 2 * 64 * 16 - 1) == 6


def test_decode_noalloc_validation(lib):
    # host-side checks run before the scratch is looked up (no GPU needed for these)
    args = lambda **kw: [kw.get("dtype", 1), kw.get("B", 2), 2, 64, 128, 128, A, A, A, A,  # noqa: E731
                         kw.get("sl", A), kw.get("o", A), ctypes.c_float(kw.get("scale", 0.1)),
                         kw.get("splits", 1), None]
    assert lib.plx_attn_decode_noalloc(*args(sl=0)) == 1
    assert lib.plx_attn_decode_noalloc(*args(o=0)) == 1
    assert lib.plx_attn_decode_noalloc(*args(B=0)) == 2
    assert lib.plx_attn_decode_noalloc(*args(scale=-1.0)) == 3
    assert lib.plx_attn_decode_noalloc(*args(dtype=0)) == 4
    assert lib.plx_attn_decode_noalloc(*args(splits=5000)) == 3


def test_missing_library_fails_loudly(monkeypatch):
    """With the HIP library absent there is no fallback: every entry point raises."""
    from attention_plx_attn_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libplx_attn.so")
    with pytest.raises(RuntimeError, match="is missing"):
        _lib.load()
    with pytest.raises(RuntimeError, match="is missing"):
        _lib.decode_num_splits(1, 16, 32768, 0)
