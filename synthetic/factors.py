"""Seeded random factor sets laid out as libmilo's arena (include/milo.h,
milo_factors): for block b, A_b^T as rank-major rows of block_len elements at
a_off[b], then B_b as rank rows of head_dim elements at b_off[b].

These are test inputs for the decode path on its own; nothing here computes
any step of the method.  Besides the packed device-side buffers the generator
returns the decoded values (what each stored element stands for) so that the
oracle can consume exactly what the kernels read.
"""
from __future__ import annotations

import numpy as np
import torch

_ELEM = {"f32": 4, "bf16": 2, "i8": 1}


def random_factor_set(n_blocks: int, T: int, d: int, storage: str, seed: int,
                      rank_range=(0, 128), a_std: float = 0.3, ranks=None):
    """Returns (tensors, A_dec, B_dec): tensors is a dict of CPU tensors
    (rank int32, a_off int64, b_off int64, arena uint8, a_scale/b_scale fp32 for
    i8); A_dec[b] is T x r fp64 and B_dec[b] is r x d fp64."""
    rng = np.random.default_rng(seed)
    if ranks is None:
        ranks = rng.integers(rank_range[0], rank_range[1] + 1, size=n_blocks)
    ranks = np.asarray(ranks, dtype=np.int32)
    e = _ELEM[storage]
    sizes = ranks.astype(np.int64) * (T + d) * e
    a_off = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
    b_off = a_off + ranks.astype(np.int64) * T * e
    total = int(sizes.sum())
    arena = np.zeros(max(total, 256), dtype=np.uint8)
    a_scale = np.zeros(n_blocks * T, dtype=np.float32) if storage == "i8" else None
    b_scale = np.zeros(n_blocks * d, dtype=np.float32) if storage == "i8" else None
    A_dec, B_dec = [], []
    for b in range(n_blocks):
        r = int(ranks[b])
        A = rng.standard_normal((T, r)) * a_std
        B = rng.standard_normal((r, d)) / np.sqrt(max(r, 1))
        if storage == "f32":
            A32, B32 = A.astype(np.float32), B.astype(np.float32)
            raw_a, raw_b = A32.T.copy().view(np.uint8), B32.view(np.uint8)
            A_dec.append(A32.astype(np.float64))
            B_dec.append(B32.astype(np.float64))
        elif storage == "bf16":
            At = torch.from_numpy(A.T.copy()).to(torch.bfloat16)
            Bt = torch.from_numpy(B.copy()).to(torch.bfloat16)
            raw_a = At.view(torch.int16).numpy().view(np.uint8)
            raw_b = Bt.view(torch.int16).numpy().view(np.uint8)
            A_dec.append(At.to(torch.float64).numpy().T.copy())
            B_dec.append(Bt.to(torch.float64).numpy())
        else:
            qa = rng.integers(-127, 128, size=(T, r)).astype(np.int8)
            qb = rng.integers(-127, 128, size=(r, d)).astype(np.int8)
            sa = (rng.uniform(0.5, 1.5, size=T) * a_std * 3 / 127).astype(np.float32)
            sb = (rng.uniform(0.5, 1.5, size=r) * 3 / np.sqrt(max(r, 1)) / 127).astype(np.float32)
            if r > 0:
                sa[rng.integers(0, T)] = 0.0          # an all-zero token row
            raw_a = qa.T.copy().view(np.uint8)
            raw_b = qb.view(np.uint8)
            a_scale[b * T:(b + 1) * T] = sa
            b_scale[b * d:b * d + r] = sb
            A_dec.append((qa.astype(np.float32) * sa[:, None]).astype(np.float64))
            B_dec.append((qb.astype(np.float32) * sb[:, None]).astype(np.float64))
        o = int(a_off[b])
        arena[o:o + raw_a.size] = raw_a.reshape(-1)
        o = int(b_off[b])
        arena[o:o + raw_b.size] = raw_b.reshape(-1)
    tensors = dict(rank=torch.from_numpy(ranks), a_off=torch.from_numpy(a_off),
                   b_off=torch.from_numpy(b_off), arena=torch.from_numpy(arena))
    if storage == "i8":
        tensors["a_scale"] = torch.from_numpy(a_scale)
        tensors["b_scale"] = torch.from_numpy(b_scale)
    return tensors, A_dec, B_dec
