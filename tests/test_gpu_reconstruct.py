"""GPU parity of milo_reconstruct on seeded factor sets in the arena layout
against the oracle's X_hat = A B (fp64), for the listed blocks only: ranks 0, 1,
around the 32-rank steps and 128; block lists in any order with repeats; fp32
and bf16 output; bf16 (MFMA path), INT8, 4-bit, 2-bit and fp32 factors."""
import numpy as np
import pytest
import torch

import oracle
from block_wise_rank_amd import Factors, milo_reconstruct
from synthetic.factors import random_factor_set

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("storage", ["bf16", "i8", "i4", "i2", "f32"])
@pytest.mark.parametrize("T", [256, 2048])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_reconstruct_listed_blocks(storage, T, out_dtype):
    d = 128
    ranks = np.array([0, 1, 31, 32, 33, 64, 100, 127, 128, 17])
    n = len(ranks)
    tens, A, B = random_factor_set(n, T, d, storage, seed=61 + T, ranks=ranks)
    f = Factors(storage, n, T, d, rank=tens["rank"].to(DEV), a_off=tens["a_off"].to(DEV),
                b_off=tens["b_off"].to(DEV), arena=tens["arena"].to(DEV))
    if storage == "i8":
        f.a_scale, f.b_scale = tens["a_scale"].to(DEV), tens["b_scale"].to(DEV)
    ids = np.array([8, 3, 0, 9, 1, 2, 4, 5, 6, 7, 8, 3], dtype=np.int32)  # any order, repeats
    out = torch.full((len(ids), T, d), float("nan"), dtype=out_dtype, device=DEV)
    milo_reconstruct(f, torch.from_numpy(ids).to(DEV), out)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    # bf16 output rounds once (2^-9 relative); the fp32 paths sum exact products in fp32
    tol = 4e-3 if out_dtype == torch.bfloat16 else 1e-5
    for i, b in enumerate(ids):
        ref = oracle.reconstruct(A[b], B[b]) if ranks[b] > 0 else np.zeros((T, d))
        den = max(np.linalg.norm(ref), 1e-300)
        err = np.linalg.norm(got[i] - ref)
        if ranks[b] == 0:
            assert err == 0.0, f"rank-0 block {b} not zero"
        else:
            assert err / den <= tol, f"{storage} T={T} block {b} (rank {ranks[b]}): rel-F {err / den:.3g}"


@pytest.mark.parametrize("storage", ["bf16", "i8", "f32"])
def test_reconstruct_at_offsets(storage):
    """milo_reconstruct_ex: each listed block's rows land at its own element
    offset of a larger buffer (gaps between them untouched), equal to the
    back-to-back reconstruction of the same list."""
    d, T = 128, 512
    ranks = np.array([5, 0, 64, 128, 33])
    n = len(ranks)
    tens, _, _ = random_factor_set(n, T, d, storage, seed=71, ranks=ranks)
    f = Factors(storage, n, T, d, rank=tens["rank"].to(DEV), a_off=tens["a_off"].to(DEV),
                b_off=tens["b_off"].to(DEV), arena=tens["arena"].to(DEV))
    if storage == "i8":
        f.a_scale, f.b_scale = tens["a_scale"].to(DEV), tens["b_scale"].to(DEV)
    ids = torch.tensor([3, 0, 4, 1, 2], dtype=torch.int32, device=DEV)
    slots = [6, 1, 3, 0, 4]                      # where each listed block goes (in blocks of T rows)
    dense = torch.empty((len(ids), T, d), dtype=torch.bfloat16, device=DEV)
    milo_reconstruct(f, ids, dense)
    big = torch.full((8, T, d), 7.0, dtype=torch.bfloat16, device=DEV)
    offs = torch.tensor([sl * T * d for sl in slots], dtype=torch.int64, device=DEV)
    milo_reconstruct(f, ids, big, out_off=offs)
    torch.cuda.synchronize()
    for i, sl in enumerate(slots):
        assert torch.equal(big[sl], dense[i]), (i, sl)
    for sl in set(range(8)) - set(slots):
        assert bool((big[sl] == 7.0).all()), sl
