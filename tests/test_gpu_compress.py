"""GPU parity of the compression path (Gram -> Jacobi eigensolve -> sigma refine ->
rank allocation -> factors) against the fp64 oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
from block_wise_rank_amd import milo_allocate_ranks
from synthetic import CONFIGS, layer_inputs
from _parity import (check_objective, check_ranks, check_reconstruction, check_sigma,
                     layer_pools, reconstruct_all, run_gpu_compress)

pytestmark = pytest.mark.gpu

DEV = "cuda"
_SVD = {}


def _case(cfg_idx, kind, storage=None, frac=None, n_pools=None):
    cfg = CONFIGS[cfg_idx]
    storage = storage or cfg.storage
    X = layer_inputs(cfg, 0, kind, device="cpu")
    pp, bud = layer_pools(cfg, frac)
    if n_pools is not None:
        pp, bud = pp[: n_pools + 1], bud[:n_pools]
        X = X[: pp[-1]]
    Xg = X.to(DEV)
    f, sig, obj, sweeps = run_gpu_compress(Xg, pp, bud, cfg.eps2, storage)
    X64 = X.to(torch.float64).numpy()
    key = (cfg_idx, kind, X64.shape[0])
    if key not in _SVD:
        _SVD[key] = oracle.svd_blocks(X64)
    comp = oracle.compress(X64, pp, bud, cfg.eps2, storage, svd=_SVD[key])
    return cfg, X64, pp, bud, f, sig, obj, sweeps, comp


@pytest.mark.parametrize("kind", ["k", "v"])
def test_config0_fp32(kind):
    cfg, X64, pp, bud, f, sig, obj, sweeps, comp = _case(0, kind)
    print(f"\n[cfg0 {kind}] sweeps {sweeps.cpu().numpy()}")
    assert (sweeps.cpu().numpy() > 0).all()
    worst = check_sigma(sig.cpu().numpy(), comp.sigma, np.sqrt(cfg.eps2))
    r_gpu = f.rank.cpu().numpy()
    nd = check_ranks(r_gpu, comp.rank, comp.sigma, pp, bud)
    xh = reconstruct_all(f).cpu().numpy()
    rec = check_reconstruction(X64, comp, r_gpu, xh, "f32")
    check_objective(obj.cpu().numpy(), sig.cpu().numpy(), r_gpu, comp.objective, comp.sigma, comp.rank, pp,
                    cfg.eps2)
    print(f"[cfg0 {kind}] sigma worst/bound {worst:.3g}, rank diffs {nd}, recon rel-F {rec:.3g}")


@pytest.mark.parametrize("kind", ["k", "v"])
def test_config1_bf16(kind):
    cfg, X64, pp, bud, f, sig, obj, sweeps, comp = _case(1, kind)
    sw = sweeps.cpu().numpy()
    print(f"\n[cfg1 {kind}] sweeps min {sw.min()} max {sw.max()} mean {sw.mean():.2f}")
    assert (sw > 0).all()
    worst = check_sigma(sig.cpu().numpy(), comp.sigma, np.sqrt(cfg.eps2))
    r_gpu = f.rank.cpu().numpy()
    nd = check_ranks(r_gpu, comp.rank, comp.sigma, pp, bud)
    xh = reconstruct_all(f).cpu().numpy()
    rec = check_reconstruction(X64, comp, r_gpu, xh, "bf16")
    check_objective(obj.cpu().numpy(), sig.cpu().numpy(), r_gpu, comp.objective, comp.sigma, comp.rank, pp,
                    cfg.eps2)
    print(f"[cfg1 {kind}] sigma worst/bound {worst:.3g}, rank diffs {nd}, recon rel-F {rec:.3g}")


def test_ranks_bit_exact_given_oracle_sigma():
    """milo_allocate_ranks on the oracle's singular values (rounded to fp32) equals
    the oracle's literal greedy on the same fp32 values, bit for bit."""
    rng = np.random.default_rng(0)
    for cfg_idx, kind in [(0, "k"), (1, "v")]:
        cfg = CONFIGS[cfg_idx]
        X = layer_inputs(cfg, 0, kind, device="cpu").to(torch.float64).numpy()
        sig, _, _ = oracle.svd_blocks(X)
        sig32 = sig.astype(np.float32)
        pp, bud = layer_pools(cfg)
        for R in [0, 1, bud[0], 3 * bud[0] // 2, 10 ** 6]:
            budgets = [R] * (len(pp) - 1)
            rank = torch.empty(X.shape[0], dtype=torch.int32, device=DEV)
            objg = torch.empty(len(pp) - 1, dtype=torch.float64, device=DEV)
            milo_allocate_ranks(torch.from_numpy(sig32).to(DEV), 128, pp, budgets, cfg.eps2, rank,
                                objg)
            torch.cuda.synchronize()
            rg = rank.cpu().numpy()
            for p in range(len(pp) - 1):
                r_o, o_o, _ = oracle.allocate(sig32[pp[p]:pp[p + 1]].astype(np.float64), R, cfg.eps2)
                assert np.array_equal(rg[pp[p]:pp[p + 1]], r_o), (cfg_idx, R, p)
                assert abs(objg[p].item() - o_o) <= 1e-12 * max(1.0, abs(o_o))
    # ties: equal singular values across blocks resolve by block index
    sig = np.tile(np.linspace(1.0, 0.0, 128, dtype=np.float32), (6, 1))
    sig[:, 100:] = 0.0
    for R in [0, 5, 6, 7, 300, 700]:
        rank = torch.empty(6, dtype=torch.int32, device=DEV)
        milo_allocate_ranks(torch.from_numpy(sig).to(DEV), 128, [0, 6], [R], 1e-4, rank)
        torch.cuda.synchronize()
        r_o, _, _ = oracle.allocate(sig.astype(np.float64), R, 1e-4)
        assert np.array_equal(rank.cpu().numpy(), r_o), R
    # random multi-pool layout with uneven pool sizes and max_rank < d
    sig = -np.sort(-rng.uniform(0, 1, size=(37, 128)).astype(np.float32), axis=1)
    pp = [0, 5, 5, 17, 37]
    bud = [100, 7, 0, 2000]
    rank = torch.empty(37, dtype=torch.int32, device=DEV)
    milo_allocate_ranks(torch.from_numpy(sig).to(DEV), 64, pp, bud, 1e-4, rank)
    torch.cuda.synchronize()
    rg = rank.cpu().numpy()
    for p in range(4):
        r_o, _, _ = oracle.allocate(sig[pp[p]:pp[p + 1], :64].astype(np.float64), bud[p], 1e-4)
        assert np.array_equal(rg[pp[p]:pp[p + 1]], r_o), p


@pytest.mark.parametrize("frac", [0.25, 0.5, 0.75])
@pytest.mark.parametrize("storage", ["bf16", "i8", "i4"])
def test_config3_budget_precision_sweep(frac, storage):
    cfg, X64, pp, bud, f, sig, obj, sweeps, comp = _case(3, "k", storage=storage, frac=frac)
    r_gpu = f.rank.cpu().numpy()
    check_ranks(r_gpu, comp.rank, comp.sigma, pp, bud)
    xh = reconstruct_all(f).cpu().numpy()
    rec = check_reconstruction(X64, comp, r_gpu, xh, storage, blocks=range(0, f.n_blocks, 3))
    full = f.n_blocks * cfg.block_len * cfg.head_dim * 2
    ratio = f.nbytes() / full
    print(f"\n[cfg3 {storage} {frac:.2f}] memory ratio vs bf16 KV {ratio:.4f}, recon rel-F {rec:.3g}")
    if storage == "i8":
        # INT8 invariants: every non-empty row of B reaches +-127; scales >= 0
        bs = f.b_scale.cpu().numpy()
        assert (bs >= 0).all() and (f.a_scale.cpu().numpy() >= 0).all()


@pytest.mark.parametrize("kind", ["k", "v"])
def test_int4_factors(kind):
    """4-bit factors on the config-1 shapes (1024-token bf16 blocks, 50% budget).

    The 4-bit path computes its factors as the fp32 storage does (the same
    products), then quantises them.  So every code and scale must equal the
    oracle's quantiser applied to the fp32 factors of a call on the same blocks
    (the code decided in fp32 on both sides): exact parity.  The quantised
    factors themselves differ from the oracle's by the eigenvector differences
    the fp32 parity allows, which move codes at rounding boundaries; the rebuilt
    blocks are therefore compared with X against the oracle's own 4-bit error."""
    from synthetic.factors import read_i4_block

    cfg = CONFIGS[1]
    X = layer_inputs(cfg, 0, kind, device="cpu")
    pp, bud = layer_pools(cfg)
    Xg = X.to(DEV)
    f32, s32, _, _ = run_gpu_compress(Xg, pp, bud, cfg.eps2, "f32")
    f4, s4, _, _ = run_gpu_compress(Xg, pp, bud, cfg.eps2, "i4")
    assert torch.equal(f32.rank, f4.rank) and torch.equal(s32, s4)
    n, T, d = X.shape
    ar32, ar4 = f32.arena.cpu().numpy(), f4.arena.cpu().numpy()
    rk = f4.rank.cpu().numpy()
    for b in range(n):
        r = int(rk[b])
        if r == 0:
            continue
        ao, bo = int(f32.a_off[b]), int(f32.b_off[b])
        A32 = ar32[ao:ao + 4 * r * T].view(np.float32).reshape(r, T)
        B32 = ar32[bo:bo + 4 * r * d].view(np.float32).reshape(r, d)
        sa, ca, _ = oracle.quant_int4_groups(A32)
        sb, cb, _ = oracle.quant_int4_groups(B32)
        ac, asc, bc, bsc = read_i4_block(ar4, int(f4.a_off[b]), int(f4.b_off[b]), r, T, d)
        assert np.array_equal(ac, ca), f"block {b}: A codes"
        assert np.array_equal(bc, cb), f"block {b}: B codes"
        assert np.array_equal(asc, sa.astype(np.float32)) and np.array_equal(bsc, sb.astype(np.float32)), b

    X64 = X.to(torch.float64).numpy()
    key = (1, kind, n)
    if key not in _SVD:
        _SVD[key] = oracle.svd_blocks(X64)
    comp = oracle.compress(X64, pp, bud, cfg.eps2, "i4", svd=_SVD[key])
    xh = reconstruct_all(f4).cpu().numpy()
    e_gpu = np.array([np.linalg.norm(xh[b] - X64[b]) / np.linalg.norm(X64[b]) for b in range(n)])
    e_ora = np.array([np.linalg.norm(oracle.reconstruct(comp.A[b], comp.B[b]) - X64[b]) / np.linalg.norm(X64[b])
                      for b in range(n)])
    print(f"\n[i4 {kind}] rel-F to X: gpu mean {e_gpu.mean():.4f} max {e_gpu.max():.4f}; "
          f"oracle mean {e_ora.mean():.4f} max {e_ora.max():.4f}; memory ratio "
          f"{f4.nbytes() / (n * T * d * 2):.4f}")
    assert (e_gpu <= 1.1 * e_ora + 2e-3).all(), np.max(e_gpu - 1.1 * e_ora)
    assert abs(e_gpu.mean() - e_ora.mean()) <= 0.05 * e_ora.mean()


@pytest.mark.parametrize("T", [192, 1088])
@pytest.mark.parametrize("storage", ["bf16", "f32", "i8"])
def test_ragged_tile_counts(T, storage):
    """Block lengths whose 32-token tile count per workgroup part is 2 mod 4
    (192: 6 tiles; 1088: a 1024-token part and a 64-token part of 2 tiles), so
    that the refine and projection tile rings run their two-tile tails."""
    from synthetic import planted_blocks
    n = 6
    X = planted_blocks(n, T, 128, (4.0, 24.0), seed=7000 + T, out_dtype="bf16")
    pp, bud = [0, n], [n * 64]
    eps2 = 1e-4
    f, sig, obj, sweeps = run_gpu_compress(X.to(DEV), pp, bud, eps2, storage)
    X64 = X.to(torch.float64).numpy()
    comp = oracle.compress(X64, pp, bud, eps2, storage)
    worst = check_sigma(sig.cpu().numpy(), comp.sigma, np.sqrt(eps2))
    r_gpu = f.rank.cpu().numpy()
    nd = check_ranks(r_gpu, comp.rank, comp.sigma, pp, bud)
    xh = reconstruct_all(f).cpu().numpy()
    rec = check_reconstruction(X64, comp, r_gpu, xh, storage)
    print(f"\n[T={T} {storage}] sigma worst/bound {worst:.3g}, rank diffs {nd}, recon rel-F {rec:.3g}")
