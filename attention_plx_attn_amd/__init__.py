"""Parallax attention forward on AMD Instinct MI355X (gfx950).

Python entry points over the C ABI of ``libplx_attn.so`` (include/plx_attn.h):

* ``prefill(q, k, v, rho, scale=None)`` -- causal prefill, [B,H,T,d] tensors;
* ``decode(q, rho, k_cache, v_cache, seqlens, scale=None, num_splits=0)`` -- one decode
  step over a contiguous per-sequence KV cache;
* ``decode_num_splits`` / ``decode_workspace_size`` -- the split plan of a decode call;
* ``decode_noalloc(q, rho, k_cache, v_cache, seqlens, out, ...)`` -- the same step for
  callers that cannot allocate (split records in the library's fixed per-GPU scratch);
* ``decode_gqa`` / ``decode_gqa_plan`` -- decode with grouped query heads (H_q = G H_kv);
* ``decode_paged`` -- decode over a paged KV cache (block pool + block table);
* ``decode_paged_gqa`` -- the same with grouped query heads;
* ``prefill_fwd`` / ``prefill_bwd`` -- the prefill with saved statistics and its backward
  (gradients of q, k, v and rho);
* ``probe(x, w_r, H, ...)`` -- the probe producer rho = gate * RoPE(RMSNorm(x W_R^T)).

All arithmetic runs in the HIP kernels; torch only supplies device memory and streams.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    PlxError,
    decode,
    decode_gqa,
    decode_gqa_plan,
    decode_noalloc,
    decode_num_splits,
    decode_paged,
    decode_paged_gqa,
    decode_workspace_size,
    header_functions,
    load,
    prefill,
    prefill_bwd,
    prefill_bwd_workspace_size,
    prefill_fwd,
    probe,
)
