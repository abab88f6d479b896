"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI and
the oracle on the same seeded inputs, and compare them."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from block_wise_rank_amd import (Factors, milo_arena_bytes, milo_compress_blocks,
                                 milo_reconstruct)
from synthetic import pool_layout

# Singular values: |sigma_gpu - sigma_oracle| <= SIGMA_REL * sigma_oracle for
# every sigma >= eps (relative 1e-3); below eps, where the gain
# log(1 + sigma^2/eps^2) ~ sigma^2/eps^2 is what the allocation reads, the bound
# is on sigma^2: |sigma_gpu^2 - sigma_oracle^2| <= 2 SIGMA_REL eps^2 (the gain to
# 2e-3; continuous with the relative bound at sigma = eps).  The eigensolve works
# on the fp32 Gram, whose backward error ~u sigma_max^2 (u = 2^-24) moves sigma^2
# by that much whatever sigma is, so no bound on sigma itself holds as sigma -> 0
# (128-token blocks have noise singular values down to ~1e-4).  Where a pool's
# budget cutoff falls below eps the selected values there are reported too.
SIGMA_REL = 1e-3
# 4-bit: the factors agree with the oracle's to ~1e-3, and an entry that close
# to a rounding boundary moves by a whole step s = max|run| / 7 (about a third
# of the run's rms): at most ~1.4% of entries, ~4% rel-Frobenius.
# 2-bit: a boundary entry moves by 2s = 2 max|run| / 3, but only three decision
# points (0 and +-2s) lie in a run's range against fourteen for 4-bit, so about
# as few entries move: the same bound (about 0.009 measured on the budget sweep).
RECON_TOL = {"f32": 1e-3, "bf16": 2e-2, "i8": 2e-2, "i4": 5e-2, "i2": 5e-2}


def run_gpu_compress(X: torch.Tensor, pool_ptr, budgets, eps2: float, storage: str):
    """X: [n, T, d] on the GPU.  Returns (factors, sigma, objective, sweeps) on the GPU."""
    n, T, d = X.shape
    arena = milo_arena_bytes(storage, T, d, pool_ptr, budgets)
    f = Factors.alloc(storage, n, T, d, arena, device=X.device)
    sigma = torch.empty((n, d), dtype=torch.float32, device=X.device)
    obj = torch.empty(len(pool_ptr) - 1, dtype=torch.float64, device=X.device)
    sweeps = torch.empty(n, dtype=torch.int32, device=X.device)
    milo_compress_blocks(X, pool_ptr, budgets, eps2, sigma, f, objective_out=obj, sweeps_out=sweeps,
                         check_convergence=True)
    torch.cuda.synchronize()
    return f, sigma, obj, sweeps


def reconstruct_all(f: Factors, out_dtype=torch.float32):
    ids = torch.arange(f.n_blocks, dtype=torch.int32, device=f.rank.device)
    out = torch.empty((f.n_blocks, f.block_len, f.head_dim), dtype=out_dtype, device=f.rank.device)
    milo_reconstruct(f, ids, out)
    torch.cuda.synchronize()
    return out


def pool_cutoffs(sig_ora: np.ndarray, pool_ptr, r_ora) -> np.ndarray:
    """Per block: the smallest singular value the oracle selects in its pool (inf
    for a pool that selects none)."""
    cut = np.full(sig_ora.shape[0], np.inf)
    for p in range(len(pool_ptr) - 1):
        lo, hi = int(pool_ptr[p]), int(pool_ptr[p + 1])
        sel = [sig_ora[b, int(r_ora[b]) - 1] for b in range(lo, hi) if int(r_ora[b]) > 0]
        if sel:
            cut[lo:hi] = min(sel)
    return cut


def check_sigma(sig_gpu: np.ndarray, sig_ora: np.ndarray, eps: float, pool_ptr=None, r_ora=None):
    """Every singular value within the bound above (relative 1e-3 from eps up, on
    sigma^2 below).
    With the pool table and the oracle's ranks, the relative error of the selected
    values below eps is printed as well."""
    sig_gpu = np.asarray(sig_gpu, dtype=np.float64)
    err = np.abs(sig_gpu - sig_ora)
    above = sig_ora >= eps
    ratio = np.where(above, err / (SIGMA_REL * np.maximum(sig_ora, eps)),
                     np.abs(sig_gpu ** 2 - sig_ora ** 2) / (2 * SIGMA_REL * eps * eps))
    worst = float(ratio.max())
    rel = err / np.maximum(sig_ora, eps)
    for lo, hi in [(0.1, np.inf), (eps, 0.1), (0.0, eps)]:
        m = (sig_ora >= lo) & (sig_ora < hi)
        if m.any():
            print(f"  sigma in [{lo:g},{hi:g}): n={int(m.sum())} max rel {rel[m].max():.3g} "
                  f"median rel {np.median(rel[m]):.3g}")
    if pool_ptr is not None:
        cut = pool_cutoffs(sig_ora, pool_ptr, r_ora)[:, None]
        m = (sig_ora >= cut) & (sig_ora < eps) & (sig_ora > 0)
        if m.any():
            r = (err / sig_ora)[m]
            print(f"  selected sigma below eps (cutoff {float(cut.min()):.3g}): n={int(m.sum())} "
                  f"max rel {r.max():.3g} median rel {np.median(r):.3g}")
    assert worst <= 1.0, f"sigma parity: worst err/bound = {worst:.3g}"
    return worst


def check_objective(obj_gpu, sig_gpu, r_gpu, obj_ora, sig_ora, r_ora, pool_ptr, eps2):
    """The GPU objective is the sum of log(1 + sigma^2/eps^2) over the ranks it handed
    out (recomputed here from its own outputs), and it is within the bound the
    sigma tolerance implies of the oracle's objective: each gain moves by at most
    |d sigma^2| / (eps^2 + sigma^2) <= 2 SIGMA_REL max(sigma, eps)^2 / (eps^2 + sigma^2)
    <= 2 SIGMA_REL, and a +-1 swap at the cutoff trades two gains whose singular
    values agree to 2 SIGMA_REL."""
    eps = np.sqrt(eps2)
    for p in range(len(pool_ptr) - 1):
        lo, hi = pool_ptr[p], pool_ptr[p + 1]
        own = sum(np.log1p(sig_gpu[b, :r_gpu[b]].astype(np.float64) ** 2 / eps2).sum()
                  for b in range(lo, hi))
        assert abs(obj_gpu[p] - own) <= 1e-12 * max(1.0, abs(own)), (p, obj_gpu[p], own)
        bound = 0.0
        for b in range(lo, hi):
            s = sig_ora[b, :int(r_gpu[b])]
            # |d sigma^2| <= 2 SIGMA_REL sigma^2 from eps up, 2 SIGMA_REL eps^2 below
            bound += (2 * SIGMA_REL * np.maximum(s, eps) ** 2 / (eps2 + s ** 2)).sum()
        n_swap = int(np.abs(np.asarray(r_gpu[lo:hi]) - np.asarray(r_ora[lo:hi])).sum())
        bound += 4 * SIGMA_REL * n_swap
        assert abs(obj_gpu[p] - obj_ora[p]) <= bound + 1e-9 * abs(obj_ora[p]), \
            (p, obj_gpu[p], obj_ora[p], bound)


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
        if r == int(comp.rank[b]):
            ref = oracle.reconstruct(comp.A[b], comp.B[b])
        else:
            ref = oracle_xhat(X64, comp, b, r, storage)
        den = np.linalg.norm(ref)
        num = np.linalg.norm(xh_gpu[b] - ref)
        rel = num / den if den > 0 else num
        worst = max(worst, rel)
        assert rel <= tol, f"block {b} (rank {r}): rel-F {rel:.3g} > {tol}"
    return worst


def layer_pools(cfg, frac=None):
    return pool_layout(cfg, frac)
