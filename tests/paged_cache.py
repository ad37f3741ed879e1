"""Scatter a contiguous decode cache into a block pool and a block table (test helper).

The pool holds the blocks of every sequence in a seeded random order, three spare blocks,
and NaN wherever no cache row was copied; table entries past a sequence's last block are
out-of-range values that the kernels must never dereference.
"""
import numpy as np
import torch


def paginate(kc: torch.Tensor, vc: torch.Tensor, seqlens: torch.Tensor, bs: int, seed: int):
    """kc, vc [B, H, L, d] (L a multiple of bs) -> k_pool, v_pool [B*L/bs + 3, H, bs, d] and
    the int32 table [B, L/bs]."""
    B, H, L, d = kc.shape
    mb = L // bs
    rng = np.random.default_rng(seed)
    nblk = B * mb + 3
    perm = rng.permutation(nblk)[: B * mb].reshape(B, mb)
    kp = torch.full((nblk, H, bs, d), float("nan"), dtype=kc.dtype)
    vp = torch.full((nblk, H, bs, vc.shape[3]), float("nan"), dtype=vc.dtype)
    table = torch.from_numpy(perm.astype(np.int32)).clone()
    for b in range(B):
        n = int(seqlens[b])
        used = (n + bs - 1) // bs
        for i in range(mb):
            if i < used:
                kp[perm[b, i]] = kc[b, :, i * bs:(i + 1) * bs]
                vp[perm[b, i]] = vc[b, :, i * bs:(i + 1) * bs]
            else:
                table[b, i] = [-7, 1 << 30, nblk][i % 3]   # never dereferenced
    return kp, vp, table
