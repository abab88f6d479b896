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
    print(f"\n[cfg0 {kind}] rotations {sweeps.cpu().numpy()}")
    assert (sweeps.cpu().numpy() > 0).all()
    worst = check_sigma(sig.cpu().numpy(), comp.sigma, np.sqrt(cfg.eps2), pp, comp.rank)
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
    print(f"\n[cfg1 {kind}] rotations min {sw.min()} max {sw.max()} mean {sw.mean():.2f}")
    assert (sw > 0).all()
    worst = check_sigma(sig.cpu().numpy(), comp.sigma, np.sqrt(cfg.eps2), pp, comp.rank)
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
    # random multi-pool layout with uneven pool sizes and max_rank < d; the last
    # pool (150 x 64 keys, and 150 x 128 below) is past what the kernel searches
    # in registers
    sig = -np.sort(-rng.uniform(0, 1, size=(187, 128)).astype(np.float32), axis=1)
    pp = [0, 5, 5, 17, 37, 187]
    bud = [100, 7, 0, 2000, 5000]
    for k in (64, 128):
        rank = torch.empty(187, dtype=torch.int32, device=DEV)
        milo_allocate_ranks(torch.from_numpy(sig).to(DEV), k, pp, bud, 1e-4, rank)
        torch.cuda.synchronize()
        rg = rank.cpu().numpy()
        for p in range(5):
            r_o, _, _ = oracle.allocate(sig[pp[p]:pp[p + 1], :k].astype(np.float64), bud[p], 1e-4)
            assert np.array_equal(rg[pp[p]:pp[p + 1]], r_o), (k, p)


def _int8_invariants(f, T, d):
    """The GPU's own INT8 factors: every row with a positive scale reaches the
    code +-127 (the absmax element), every row with a zero scale is all zero."""
    ar = f.arena.cpu().numpy()
    a_sc, b_sc = f.a_scale.cpu().numpy(), f.b_scale.cpu().numpy()
    rk = f.rank.cpu().numpy()
    for b in range(f.n_blocks):
        r = int(rk[b])
        if r == 0:
            continue
        ao, bo = int(f.a_off[b]), int(f.b_off[b])
        A8 = ar[ao:ao + r * T].view(np.int8).reshape(r, T).astype(np.int32)
        B8 = ar[bo:bo + r * d].view(np.int8).reshape(r, d).astype(np.int32)
        for codes, sc in ((A8.T, a_sc[b * T:(b + 1) * T]), (B8, b_sc[b * d:b * d + r])):
            top = np.abs(codes).max(axis=1)
            assert (sc >= 0).all(), b
            assert (top[sc > 0] == 127).all(), f"block {b}: a row with a positive scale misses +-127"
            assert (top[sc == 0] == 0).all(), f"block {b}: a zero-scale row holds codes"


@pytest.mark.parametrize("frac", [0.25, 0.5, 0.75])
@pytest.mark.parametrize("storage", ["bf16", "i8", "i4", "i2"])
def test_config3_budget_precision_sweep(frac, storage):
    cfg, X64, pp, bud, f, sig, obj, sweeps, comp = _case(3, "k", storage=storage, frac=frac)
    r_gpu = f.rank.cpu().numpy()
    check_sigma(sig.cpu().numpy(), comp.sigma, np.sqrt(cfg.eps2), pp, comp.rank)
    check_ranks(r_gpu, comp.rank, comp.sigma, pp, bud)
    xh = reconstruct_all(f).cpu().numpy()
    rec = check_reconstruction(X64, comp, r_gpu, xh, storage)
    full = f.n_blocks * cfg.block_len * cfg.head_dim * 2
    ratio = f.nbytes() / full
    print(f"\n[cfg3 {storage} {frac:.2f}] memory ratio vs bf16 KV {ratio:.4f}, recon rel-F {rec:.3g}")
    if storage == "i8":
        _int8_invariants(f, cfg.block_len, cfg.head_dim)


@pytest.mark.parametrize("kind", ["k", "v"])
def test_int8_codes(kind):
    """INT8 factors on the config-1 shapes (1024-token bf16 blocks, 50% budget)
    against the oracle's quantiser, code by code.

    B: the INT8 path quantises the same fp32 eigenvector rows the fp32 storage
    stores, with the code decided in fp32 on both sides, so every B code and
    scale must equal the oracle's quantiser applied to the fp32 factors of a call
    on the same blocks.  A = X B~^T is formed from the dequantised B~ (codes x
    scale): the oracle quantises the exact product (fp64) per token row; the GPU
    sums in fp32, so a code may differ by one step where the product lies within
    fp32 rounding of a rounding boundary, and the scales agree to fp32 accuracy."""
    cfg = CONFIGS[1]
    X = layer_inputs(cfg, 0, kind, device="cpu")
    pp, bud = layer_pools(cfg)
    Xg = X.to(DEV)
    f32, s32, _, _ = run_gpu_compress(Xg, pp, bud, cfg.eps2, "f32")
    f8, s8, _, _ = run_gpu_compress(Xg, pp, bud, cfg.eps2, "i8")
    assert torch.equal(f32.rank, f8.rank) and torch.equal(s32, s8)
    n, T, d = X.shape
    X64 = X.to(torch.float64).numpy()
    ar32, ar8 = f32.arena.cpu().numpy(), f8.arena.cpu().numpy()
    a_sc, b_sc = f8.a_scale.cpu().numpy(), f8.b_scale.cpu().numpy()
    rk = f8.rank.cpu().numpy()
    n_off = n_codes = 0
    worst_scale = 0.0
    for b in range(n):
        r = int(rk[b])
        if r == 0:
            continue
        B32 = ar32[int(f32.b_off[b]):int(f32.b_off[b]) + 4 * r * d].view(np.float32).reshape(r, d)
        sb, cb, _ = oracle.quant_int8_rows(B32)
        bo = int(f8.b_off[b])
        B8 = ar8[bo:bo + r * d].view(np.int8).reshape(r, d)
        assert np.array_equal(B8, cb), f"block {b}: B codes"
        assert np.array_equal(b_sc[b * d:b * d + r], sb.astype(np.float32)), f"block {b}: B scales"
        A_ref = (X64[b] @ B8.T.astype(np.float64)) * b_sc[b * d:b * d + r].astype(np.float64)  # T x r
        sa, ca, _ = oracle.quant_int8_rows(A_ref)
        ao = int(f8.a_off[b])
        A8 = ar8[ao:ao + r * T].view(np.int8).reshape(r, T).T
        diff = np.abs(A8.astype(np.int32) - ca.astype(np.int32))
        assert diff.max() <= 1, f"block {b}: A code off by {diff.max()}"
        n_off += int((diff != 0).sum())
        n_codes += diff.size
        ga = a_sc[b * T:(b + 1) * T].astype(np.float64)
        worst_scale = max(worst_scale, float((np.abs(ga - sa) / np.maximum(sa, 1e-30)).max()))
    print(f"\n[i8 {kind}] A codes one step off: {n_off} of {n_codes}; worst A scale rel err {worst_scale:.3g}")
    assert worst_scale <= 1e-5
    assert n_off <= 1e-3 * n_codes
    _int8_invariants(f8, T, d)


@pytest.mark.parametrize("path", ["jacobi", "qr"])
def test_compress_edge_cases(path):
    """Degenerate blocks through the whole compression, fp32 storage, against the
    oracle: an all-zero block, a rank-1 block, a block with orthonormal columns
    (every singular value 1, so the singular subspaces are not unique), and the
    same planted blocks at x1e-3, x1 and x1e3 in pools of their own (the method
    is scale-invariant: equal ranks, singular values and relative errors).  The
    ten blocks alone take the Jacobi eigensolve; with enough planted pools after
    them (more than eight blocks per CU) the same call takes Householder + QR."""
    from synthetic import planted_blocks
    T, d = 256, 128
    P = planted_blocks(2, T, d, (4.0, 32.0), seed=8101, out_dtype="f64")
    g = torch.Generator().manual_seed(8102)
    a = torch.randn(T, generator=g, dtype=torch.float64)
    v = torch.randn(d, generator=g, dtype=torch.float64)
    rank1 = 0.7 * torch.outer(a / a.norm(), v / v.norm())
    Q, _ = torch.linalg.qr(torch.randn(T, d, generator=g, dtype=torch.float64))
    blocks = [torch.zeros(T, d, dtype=torch.float64), rank1, P[0], Q,
              1e-3 * P[0], 1e-3 * P[1], 1e3 * P[0], 1e3 * P[1], P[0], P[1]]
    scale = np.array([1, 1, 1, 1, 1e-3, 1e-3, 1e3, 1e3, 1, 1], dtype=np.float64)
    X = torch.stack(blocks).to(torch.float32)
    pp, bud = [0, 3, 4, 6, 8, 10], [100, 50, 128, 128, 128]
    eps2 = 1e-4
    Xg, ppg, budg = X, pp, bud
    if path == "qr":
        n_cus = torch.cuda.get_device_properties(0).multi_processor_count
        n_pad = 64 * (8 * n_cus // 64 + 1)
        pad = planted_blocks(n_pad, T, d, (4.0, 32.0), seed=8103, out_dtype="f32")
        Xg = torch.cat([X, pad])
        ppg = pp + [10 + 64 * (i + 1) for i in range(n_pad // 64)]
        budg = bud + [64 * 64] * (n_pad // 64)
    f, sig, obj, sweeps = run_gpu_compress(Xg.to(DEV), ppg, budg, eps2, "f32")
    sw = sweeps.cpu().numpy()
    assert (sw >= 0).all(), "no block may stop at an iteration cap"
    assert (sw[[2, 4, 5, 6, 7, 8, 9]] > 0).all()
    if path == "qr":
        assert sw[0] == 0  # the zero Gram is diagonal once reduced: no QR step
    sig, obj, sw = sig[:10], obj[:5], sw[:10]
    X64 = X.to(torch.float64).numpy()
    comp = oracle.compress(X64, pp, bud, eps2, "f32")
    sg = sig.cpu().numpy().astype(np.float64)
    worst = check_sigma(sg / scale[:, None], comp.sigma / scale[:, None], np.sqrt(eps2), pp, comp.rank)
    assert (sg[0] == 0).all(), "zero block: singular values"
    r_gpu = f.rank.cpu().numpy()[:10]
    check_ranks(r_gpu, comp.rank, comp.sigma, pp, bud)
    assert list(r_gpu[:4]) == [0, 1, 99, 50]
    assert np.array_equal(r_gpu[4:6], r_gpu[8:10]) and np.array_equal(r_gpu[6:8], r_gpu[8:10])
    xh = reconstruct_all(f)[:10].cpu().numpy().astype(np.float64)
    assert (xh[0] == 0).all()
    rec = check_reconstruction(X64, comp, r_gpu, xh, "f32", blocks=[0, 1, 2, 4, 5, 6, 7, 8, 9])
    # orthonormal columns: any 50 of the equal singular directions are a best
    # rank-50 approximation; what is unique is the residual (78 of 128 unit
    # values, Eckart-Young) and that the factors are X projected on an
    # orthonormal basis (B B^T = I, A = X B^T)
    res = np.sum((xh[3] - X64[3]) ** 2)
    assert abs(res - np.sum(comp.sigma[3, 50:] ** 2)) <= 1e-4 * 128, res
    ar = f.arena.cpu().numpy()
    B = ar[int(f.b_off[3]):int(f.b_off[3]) + 4 * 50 * d].view(np.float32).reshape(50, d).astype(np.float64)
    A = ar[int(f.a_off[3]):int(f.a_off[3]) + 4 * 50 * T].view(np.float32).reshape(50, T).T.astype(np.float64)
    assert np.abs(B @ B.T - np.eye(50)).max() <= 1e-5
    assert np.abs(A - X64[3] @ B.T).max() <= 1e-5
    print(f"\n[edge] sigma worst/bound {worst:.3g}, ranks {list(r_gpu)}, recon rel-F {rec:.3g}, "
          f"orthonormal-block residual {res:.4f}")


def test_eigensolve_paths_large_and_small_launch():
    """The eigensolve has two paths: a launch with more than eight blocks per CU
    takes Householder tridiagonalisation and QR steps (64 blocks per wave, the
    recorded rotations applied in a second kernel); a smaller launch takes the
    Jacobi eigensolve, one workgroup per block.  Planted 256-token blocks in pools
    of 64, enough of them for the first path: the first and last pools against
    the oracle (sigma, ranks, fp32 reconstruction), and the first pool
    compressed alone (the second path) must give the same singular values to
    within a tenth of their tolerance."""
    from synthetic import planted_blocks
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_pools = 8 * n_cus // 64 + 1
    n, T = 64 * n_pools, 256
    X = planted_blocks(n, T, 128, (4.0, 32.0), seed=8301, out_dtype="bf16")
    pp, bud = [64 * i for i in range(n_pools + 1)], [64 * 48] * n_pools
    eps2 = 1e-4
    f, sig, obj, rots = run_gpu_compress(X.to(DEV), pp, bud, eps2, "f32")
    r = rots.cpu().numpy()
    assert (r > 0).all()
    X64 = X.to(torch.float64).numpy()
    xh_all = reconstruct_all(f).cpu().numpy()
    for pool in (0, n_pools - 1):
        lo, hi = pp[pool], pp[pool + 1]
        comp = oracle.compress(X64[lo:hi], [0, hi - lo], [bud[pool]], eps2, "f32")
        check_sigma(sig[lo:hi].cpu().numpy(), comp.sigma, np.sqrt(eps2), [0, hi - lo], comp.rank)
        r_gpu = f.rank[lo:hi].cpu().numpy()
        check_ranks(r_gpu, comp.rank, comp.sigma, [0, hi - lo], [bud[pool]])
        check_reconstruction(X64[lo:hi], comp, r_gpu, xh_all[lo:hi], "f32")
    f1, sig1, _, rots1 = run_gpu_compress(X[:64].to(DEV), [0, 64], [bud[0]], eps2, "f32")
    a, b = sig[:64].double().cpu().numpy(), sig1.double().cpu().numpy()
    assert np.max(np.abs(a - b) / np.maximum(b, np.sqrt(eps2))) < 1e-4
    print(f"\n[eigensolve paths] {n} blocks: {r.mean():.0f} QR rotations per block; "
          f"64 blocks: {rots1.double().mean().item():.0f} Jacobi rotations per block")


def test_block_len_128():
    """The smallest block length: 128 tokens, so k = min(T, d) = T = d."""
    from synthetic import planted_blocks
    n, T = 8, 128
    X = planted_blocks(n, T, 128, (4.0, 24.0), seed=8201, out_dtype="bf16")
    pp, bud = [0, 5, 8], [5 * 64, 3 * 64]
    eps2 = 1e-4
    for storage in ("bf16", "f32", "i8", "i4", "i2"):
        f, sig, obj, sweeps = run_gpu_compress(X.to(DEV), pp, bud, eps2, storage)
        X64 = X.to(torch.float64).numpy()
        comp = oracle.compress(X64, pp, bud, eps2, storage)
        worst = check_sigma(sig.cpu().numpy(), comp.sigma, np.sqrt(eps2), pp, comp.rank)
        r_gpu = f.rank.cpu().numpy()
        check_ranks(r_gpu, comp.rank, comp.sigma, pp, bud)
        xh = reconstruct_all(f).cpu().numpy()
        if storage in ("i4", "i2"):
            # A 128-token block puts a few factor entries within rounding distance
            # of a 2-bit decision point (0, +-2s), where a flip moves the entry by
            # 2s = 2 max|run| / 3: the rebuilt block can then differ from the
            # oracle's by several percent while both are equally far from X.  So
            # the low-bit blocks are compared with X against the oracle's own
            # low-bit error (the codes themselves are checked exactly against the
            # oracle's quantiser in the grouped-factor tests).
            e_gpu = np.array([np.linalg.norm(xh[b] - X64[b]) / np.linalg.norm(X64[b]) for b in range(n)])
            e_ora = np.array([np.linalg.norm(oracle.reconstruct(comp.A[b], comp.B[b]) - X64[b]) /
                              np.linalg.norm(X64[b]) for b in range(n)])
            assert (e_gpu <= 1.1 * e_ora + 2e-3).all(), np.max(e_gpu - 1.1 * e_ora)
            rec = float(np.max(np.abs(e_gpu - e_ora)))
        else:
            rec = check_reconstruction(X64, comp, r_gpu, xh, storage)
        check_objective(obj.cpu().numpy(), sig.cpu().numpy(), r_gpu, comp.objective, comp.sigma, comp.rank,
                        pp, eps2)
        print(f"\n[T=128 {storage}] sigma worst/bound {worst:.3g}, recon rel-F {rec:.3g}")


@pytest.mark.parametrize("storage", ["i4", "i2"])
@pytest.mark.parametrize("kind", ["k", "v"])
def test_grouped_lowbit_factors(kind, storage):
    """4- and 2-bit factors on the config-1 shapes (1024-token bf16 blocks, 50%
    budget).

    The low-bit paths compute their factors as the fp32 storage does (the same
    products), then quantise them.  So every code and scale must equal the
    oracle's quantiser applied to the fp32 factors of a call on the same blocks
    (the code decided in fp32 on both sides): exact parity.  The quantised
    factors themselves differ from the oracle's by the eigenvector differences
    the fp32 parity allows, which move codes at decision boundaries; the rebuilt
    blocks are therefore compared with X against the oracle's own low-bit error."""
    from synthetic.factors import read_i2_block, read_i4_block

    quant = oracle.quant_int4_groups if storage == "i4" else oracle.quant_int2_groups
    read_block = read_i4_block if storage == "i4" else read_i2_block
    cfg = CONFIGS[1]
    X = layer_inputs(cfg, 0, kind, device="cpu")
    pp, bud = layer_pools(cfg)
    Xg = X.to(DEV)
    f32, s32, _, _ = run_gpu_compress(Xg, pp, bud, cfg.eps2, "f32")
    f4, s4, _, _ = run_gpu_compress(Xg, pp, bud, cfg.eps2, storage)
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
        sa, ca, _ = quant(A32)
        sb, cb, _ = quant(B32)
        ac, asc, bc, bsc = read_block(ar4, int(f4.a_off[b]), int(f4.b_off[b]), r, T, d)
        assert np.array_equal(ac, ca), f"block {b}: A codes"
        assert np.array_equal(bc, cb), f"block {b}: B codes"
        assert np.array_equal(asc, sa.astype(np.float32)) and np.array_equal(bsc, sb.astype(np.float32)), b

    X64 = X.to(torch.float64).numpy()
    key = (1, kind, n)
    if key not in _SVD:
        _SVD[key] = oracle.svd_blocks(X64)
    comp = oracle.compress(X64, pp, bud, cfg.eps2, storage, svd=_SVD[key])
    xh = reconstruct_all(f4).cpu().numpy()
    e_gpu = np.array([np.linalg.norm(xh[b] - X64[b]) / np.linalg.norm(X64[b]) for b in range(n)])
    e_ora = np.array([np.linalg.norm(oracle.reconstruct(comp.A[b], comp.B[b]) - X64[b]) / np.linalg.norm(X64[b])
                      for b in range(n)])
    print(f"\n[{storage} {kind}] rel-F to X: gpu mean {e_gpu.mean():.4f} max {e_gpu.max():.4f}; "
          f"oracle mean {e_ora.mean():.4f} max {e_ora.max():.4f}; memory ratio "
          f"{f4.nbytes() / (n * T * d * 2):.4f}")
    assert (e_gpu <= 1.1 * e_ora + 2e-3).all(), np.max(e_gpu - 1.1 * e_ora)
    assert abs(e_gpu.mean() - e_ora.mean()) <= 0.05 * e_ora.mean()


@pytest.mark.parametrize("storage", ["i4", "i2"])
def test_grouped_lowbit_factors_fp32_input(storage):
    """The fp32-input projection (X split into three bf16 terms) into 4- and 2-bit
    factors, on the config-0 shapes (256-token fp32 blocks, K and V of the planted
    spectra): every code and scale equals the oracle's quantiser applied to the
    fp32 factors a call with fp32 storage writes for the same blocks."""
    from synthetic.factors import read_i2_block, read_i4_block

    quant = oracle.quant_int4_groups if storage == "i4" else oracle.quant_int2_groups
    read_block = read_i4_block if storage == "i4" else read_i2_block
    cfg = CONFIGS[0]
    pp, bud = layer_pools(cfg)
    for kind in ("k", "v"):
        X = layer_inputs(cfg, 0, kind, device=DEV)
        assert X.dtype == torch.float32
        f32, s32, _, _ = run_gpu_compress(X, pp, bud, cfg.eps2, "f32")
        fq, sq, _, _ = run_gpu_compress(X, pp, bud, cfg.eps2, storage)
        assert torch.equal(f32.rank, fq.rank) and torch.equal(s32, sq)
        n, T, d = X.shape
        ar32, arq = f32.arena.cpu().numpy(), fq.arena.cpu().numpy()
        rk = fq.rank.cpu().numpy()
        for b in range(n):
            r = int(rk[b])
            if r == 0:
                continue
            ao, bo = int(f32.a_off[b]), int(f32.b_off[b])
            A32 = ar32[ao:ao + 4 * r * T].view(np.float32).reshape(r, T)
            B32 = ar32[bo:bo + 4 * r * d].view(np.float32).reshape(r, d)
            sa, ca, _ = quant(A32)
            sb, cb, _ = quant(B32)
            ac, asc, bc, bsc = read_block(arq, int(fq.a_off[b]), int(fq.b_off[b]), r, T, d)
            assert np.array_equal(ac, ca), f"{kind} block {b}: A codes"
            assert np.array_equal(bc, cb), f"{kind} block {b}: B codes"
            assert np.array_equal(asc, sa.astype(np.float32)) and np.array_equal(bsc, sb.astype(np.float32))


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
    worst = check_sigma(sig.cpu().numpy(), comp.sigma, np.sqrt(eps2), pp, comp.rank)
    r_gpu = f.rank.cpu().numpy()
    nd = check_ranks(r_gpu, comp.rank, comp.sigma, pp, bud)
    xh = reconstruct_all(f).cpu().numpy()
    rec = check_reconstruction(X64, comp, r_gpu, xh, storage)
    print(f"\n[T={T} {storage}] sigma worst/bound {worst:.3g}, rank diffs {nd}, recon rel-F {rec:.3g}")
