"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI and
the oracle on the same seeded inputs, and compare them."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from block_wise_rank_amd import (Factors, milo_arena_bytes, milo_compress_blocks,
                                 milo_reconstruct)
from synthetic import pool_layout

# |sigma_gpu - sigma_oracle| <= SIGMA_REL * max(sigma_oracle, eps): relative 1e-3
# for every singular value above eps (all the ones the allocation can pick),
# absolute 1e-3 * eps below it, where log(1 + sigma^2/eps^2) is flat.
SIGMA_REL = 1e-3
RECON_TOL = {"f32": 1e-3, "bf16": 2e-2, "i8": 2e-2}


def run_gpu_compress(X: torch.Tensor, pool_ptr, budgets, eps2: float, storage: str):
    """X: [n, T, d] on the GPU.  Returns (factors, sigma, objective, sweeps) on the GPU."""
    n, T, d = X.shape
    arena = milo_arena_bytes(storage, T, d, pool_ptr, budgets)
    f = Factors.alloc(storage, n, T, d, arena, device=X.device)
    sigma = torch.empty((n, d), dtype=torch.float32, device=X.device)
    obj = torch.empty(len(pool_ptr) - 1, dtype=torch.float64, device=X.device)
    sweeps = torch.empty(n, dtype=torch.int32, device=X.device)
    milo_compress_blocks(X, pool_ptr, budgets, eps2, sigma, f, objective_out=obj, sweeps_out=sweeps)
    torch.cuda.synchronize()
    return f, sigma, obj, sweeps


def reconstruct_all(f: Factors, out_dtype=torch.float32):
    ids = torch.arange(f.n_blocks, dtype=torch.int32, device=f.rank.device)
    out = torch.empty((f.n_blocks, f.block_len, f.head_dim), dtype=out_dtype, device=f.rank.device)
    milo_reconstruct(f, ids, out)
    torch.cuda.synchronize()
    return out


def check_sigma(sig_gpu: np.ndarray, sig_ora: np.ndarray, eps: float):
    bound = SIGMA_REL * np.maximum(sig_ora, eps)
    err = np.abs(sig_gpu - sig_ora)
    worst = float((err / bound).max())
    assert worst <= 1.0, f"sigma parity: worst err/bound = {worst:.3g}"
    return worst


def check_ranks(r_gpu: np.ndarray, r_ora: np.ndarray, sig_ora: np.ndarray, pool_ptr, budgets):
    """Budget spent exactly; ranks equal the oracle's except +-1 swaps at the
    budget cutoff, where the swapped singular values tie to within the sigma
    tolerance (the selection there is not unique at fp32 accuracy)."""
    k = sig_ora.shape[1]
    n_diff = 0
    for p in range(len(pool_ptr) - 1):
        lo, hi = pool_ptr[p], pool_ptr[p + 1]
        want = min(int(budgets[p]), (hi - lo) * k)
        assert int(r_gpu[lo:hi].sum()) == want, f"pool {p}: budget not spent exactly"
        diff = r_gpu[lo:hi] - r_ora[lo:hi]
        if not diff.any():
            continue
        assert np.abs(diff).max() <= 1, f"pool {p}: rank differs by more than one"
        # the oracle's cutoff value: the smallest selected sigma of the pool
        sel = [sig_ora[b, r_ora[b] - 1] for b in range(lo, hi) if r_ora[b] > 0]
        cut = min(sel)
        for b in np.nonzero(diff)[0] + lo:
            i = min(r_gpu[b], r_ora[b])
            assert abs(sig_ora[b, i] - cut) <= 2 * SIGMA_REL * cut, \
                f"block {b}: rank swap away from the cutoff ({sig_ora[b, i]} vs {cut})"
        n_diff += int(np.abs(diff).sum())
    return n_diff


def oracle_xhat(X64: np.ndarray, comp: oracle.Compressed, b: int, r: int, storage: str):
    """The oracle's stored reconstruction of block b at rank r (its own SVD)."""
    A, B = oracle.project(X64[b], comp.V[b], r)
    A, B = oracle.store(A, B, storage)
    return oracle.reconstruct(A, B)


def check_reconstruction(X64, comp, r_gpu, xh_gpu: np.ndarray, storage: str, blocks=None):
    """rel-Frobenius of the GPU reconstruction against the oracle's, per block.  When
    the GPU rank differs from the oracle's (a cutoff swap) the oracle's own
    reconstruction at that rank is the reference."""
    tol = RECON_TOL[storage]
    worst = 0.0
    for b in (range(len(r_gpu)) if blocks is None else blocks):
        r = int(r_gpu[b])
        ref = comp_xhat_cache(X64, comp, b, r, storage)
        den = np.linalg.norm(ref)
        num = np.linalg.norm(xh_gpu[b] - ref)
        rel = num / den if den > 0 else num
        worst = max(worst, rel)
        assert rel <= tol, f"block {b} (rank {r}): rel-F {rel:.3g} > {tol}"
    return worst


_cache = {}


def comp_xhat_cache(X64, comp, b, r, storage):
    key = (id(comp), b, r, storage)
    if key not in _cache:
        if r == int(comp.rank[b]):
            _cache[key] = oracle.reconstruct(comp.A[b], comp.B[b])
        else:
            _cache[key] = oracle_xhat(X64, comp, b, r, storage)
    return _cache[key]


def layer_pools(cfg, frac=None):
    return pool_layout(cfg, frac)
