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
I4_GROUP = 32


def pack_i4(codes: np.ndarray) -> np.ndarray:
    """Rows of 4-bit codes in [-8, 7] -> bytes, element 2k in the low nibble of
    byte k (the arena's nibble order)."""
    c = (codes.astype(np.int16) & 0xF).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_i4(raw: np.ndarray, n: int) -> np.ndarray:
    """Inverse of pack_i4 for rows of n codes."""
    raw = raw.astype(np.uint8)
    lo = (raw & 0xF).astype(np.int16)
    hi = (raw >> 4).astype(np.int16)
    out = np.empty(raw.shape[:-1] + (n,), dtype=np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return np.where(out >= 8, out - 16, out).astype(np.int8)


def pack_i2(codes: np.ndarray) -> np.ndarray:
    """Rows of 2-bit codes in 0..3 -> bytes, element 4k + j in bits 2j, 2j + 1 of
    byte k (the arena's order)."""
    c = (codes.astype(np.uint8) & 3)
    return (c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)).astype(np.uint8)


def unpack_i2(raw: np.ndarray, n: int) -> np.ndarray:
    """Inverse of pack_i2 for rows of n codes."""
    raw = raw.astype(np.uint8)
    out = np.empty(raw.shape[:-1] + (n,), dtype=np.uint8)
    for j in range(4):
        out[..., j::4] = (raw >> (2 * j)) & 3
    return out


def i2_rank_bytes(T: int, d: int):
    """Bytes one rank takes in a block's A part and B part (2-bit codes + fp32 scales)."""
    return T // 4 + 4 * (T // I4_GROUP), d // 4 + 4 * (d // I4_GROUP)


def read_i2_block(arena: np.ndarray, a_off: int, b_off: int, r: int, T: int, d: int):
    """(A codes [r, T], A scales [r, T/32], B codes [r, d], B scales [r, d/32]) of a block."""
    a_codes = unpack_i2(arena[a_off:a_off + r * T // 4].reshape(r, T // 4), T)
    o = a_off + r * T // 4
    a_sc = arena[o:o + 4 * r * (T // I4_GROUP)].view(np.float32).reshape(r, T // I4_GROUP)
    b_codes = unpack_i2(arena[b_off:b_off + r * d // 4].reshape(r, d // 4), d)
    o = b_off + r * d // 4
    b_sc = arena[o:o + 4 * r * (d // I4_GROUP)].view(np.float32).reshape(r, d // I4_GROUP)
    return a_codes, a_sc, b_codes, b_sc


def i4_rank_bytes(T: int, d: int):
    """Bytes one rank takes in a block's A part and B part (codes + fp32 scales)."""
    return T // 2 + 4 * (T // I4_GROUP), d // 2 + 4 * (d // I4_GROUP)


def read_i4_block(arena: np.ndarray, a_off: int, b_off: int, r: int, T: int, d: int):
    """(A codes [r, T], A scales [r, T/32], B codes [r, d], B scales [r, d/32]) of a block."""
    a_codes = unpack_i4(arena[a_off:a_off + r * T // 2].reshape(r, T // 2), T)
    o = a_off + r * T // 2
    a_sc = arena[o:o + 4 * r * (T // I4_GROUP)].view(np.float32).reshape(r, T // I4_GROUP)
    b_codes = unpack_i4(arena[b_off:b_off + r * d // 2].reshape(r, d // 2), d)
    o = b_off + r * d // 2
    b_sc = arena[o:o + 4 * r * (d // I4_GROUP)].view(np.float32).reshape(r, d // I4_GROUP)
    return a_codes, a_sc, b_codes, b_sc


def random_factor_set(n_blocks: int, T: int, d: int, storage: str, seed: int,
                      rank_range=(0, 128), a_std: float = 0.3, ranks=None):
    """Returns (tensors, A_dec, B_dec): tensors is a dict of CPU tensors
    (rank int32, a_off int64, b_off int64, arena uint8, a_scale/b_scale fp32 for
    i8); A_dec[b] is T x r fp64 and B_dec[b] is r x d fp64."""
    rng = np.random.default_rng(seed)
    if ranks is None:
        ranks = rng.integers(rank_range[0], rank_range[1] + 1, size=n_blocks)
    ranks = np.asarray(ranks, dtype=np.int32)
    if storage == "i4":
        abpr, bbpr = i4_rank_bytes(T, d)
    elif storage == "i2":
        abpr, bbpr = i2_rank_bytes(T, d)
    else:
        abpr, bbpr = T * _ELEM[storage], d * _ELEM[storage]
    sizes = ranks.astype(np.int64) * (abpr + bbpr)
    a_off = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
    b_off = a_off + ranks.astype(np.int64) * abpr
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
        elif storage == "i4":
            # codes in [-7, 7], one positive scale per 32 elements of a row (some
            # runs all zero with a zero scale, as the quantiser leaves them)
            ca = rng.integers(-7, 8, size=(r, T)).astype(np.int8)
            cb = rng.integers(-7, 8, size=(r, d)).astype(np.int8)
            sa = (rng.uniform(0.5, 1.5, size=(r, T // I4_GROUP)) * a_std * 3 / 7).astype(np.float32)
            sb = (rng.uniform(0.5, 1.5, size=(r, d // I4_GROUP)) * 3 / np.sqrt(max(r, 1)) / 7).astype(np.float32)
            if r > 0:
                i, g = rng.integers(0, r), rng.integers(0, T // I4_GROUP)
                ca[i, g * I4_GROUP:(g + 1) * I4_GROUP] = 0
                sa[i, g] = 0.0
            raw_a = np.concatenate([pack_i4(ca).reshape(-1), sa.reshape(-1).view(np.uint8)])
            raw_b = np.concatenate([pack_i4(cb).reshape(-1), sb.reshape(-1).view(np.uint8)])
            A_dec.append((ca.astype(np.float32) * np.repeat(sa, I4_GROUP, axis=1)).astype(np.float64).T.copy())
            B_dec.append((cb.astype(np.float32) * np.repeat(sb, I4_GROUP, axis=1)).astype(np.float64))
        elif storage == "i2":
            # codes in 0..3 for the levels (2c - 3) s, one positive scale per 32
            # elements of a row (some runs all code 2 with a zero scale, as the
            # quantiser leaves an all-zero run)
            ca = rng.integers(0, 4, size=(r, T)).astype(np.uint8)
            cb = rng.integers(0, 4, size=(r, d)).astype(np.uint8)
            sa = (rng.uniform(0.5, 1.5, size=(r, T // I4_GROUP)) * a_std / 3).astype(np.float32)
            sb = (rng.uniform(0.5, 1.5, size=(r, d // I4_GROUP)) / np.sqrt(max(r, 1)) / 3).astype(np.float32)
            if r > 0:
                i, g = rng.integers(0, r), rng.integers(0, T // I4_GROUP)
                ca[i, g * I4_GROUP:(g + 1) * I4_GROUP] = 2
                sa[i, g] = 0.0
            raw_a = np.concatenate([pack_i2(ca).reshape(-1), sa.reshape(-1).view(np.uint8)])
            raw_b = np.concatenate([pack_i2(cb).reshape(-1), sb.reshape(-1).view(np.uint8)])
            lv_a = (2 * ca.astype(np.int16) - 3).astype(np.float32)
            lv_b = (2 * cb.astype(np.int16) - 3).astype(np.float32)
            A_dec.append((lv_a * np.repeat(sa, I4_GROUP, axis=1)).astype(np.float64).T.copy())
            B_dec.append((lv_b * np.repeat(sb, I4_GROUP, axis=1)).astype(np.float64))
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
