"""GPU parity at the full sizes of the benchmark workloads, in the launch
configuration the benchmark uses, on outputs the oracle computes one
(sequence, KV head) unit at a time.

For one layer of a workload the GPU compresses every K and V block with the
benchmark's pool layout (one pool per sequence, KV head and K/V, half of the
ranks) and decodes the step with the default split.  For two sampled units the
oracle compresses the same seeded inputs (the unit's K pool and V pool, copied
from the device where the generator made them) and decodes the unit's query
heads.  Compared: every singular value and rank of the two pools, their
objectives, the reconstruction of sampled blocks and the attention output of the
unit's query heads (queries x300, so the softmax is exercised), to the same
tolerances as the small cases.

  * long context, Qwen2.5-3B-shaped: 16 sequences x 2 KV heads x 64 blocks of 2048
    tokens, 16 query heads (GQA 8:1);
  * Qwen2.5-7B-shaped stack with selection and tail: 8 sequences x 4 KV heads x 64
    blocks of 1024 tokens, 28 query heads (GQA 7:1), 8 selected blocks per sequence
    and a 256-token uncompressed tail;
  * the long-context layer again with 4- and 2-bit factors (one unit each).
"""
import numpy as np
import pytest
import torch

import oracle
from block_wise_rank_amd import milo_decode_attention, milo_reconstruct
from synthetic import CONFIGS, layer_inputs, queries, selection
from synthetic.planted import tail_inputs
from _parity import (RECON_TOL, check_objective, check_ranks, check_sigma, layer_pools,
                     run_gpu_compress)

pytestmark = pytest.mark.gpu
DEV = "cuda"
Q_SCALE = 300.0


def _unit_blocks(cfg, s, h):
    lo = (s * cfg.n_kv_heads + h) * cfg.blocks_per_seq
    return lo, lo + cfg.blocks_per_seq


def _check_unit(cfg, s, h, X, comp_gpu, sig_gpu, obj_gpu, storage):
    """Oracle compression of one unit's pool against the GPU's; returns the oracle's
    reconstructed blocks of the pool."""
    lo, hi = _unit_blocks(cfg, s, h)
    X64 = X[lo:hi].to(torch.float64).cpu().numpy()
    R = cfg.budget()
    ora = oracle.compress(X64, [0, hi - lo], [R], cfg.eps2, storage)
    sg = sig_gpu[lo:hi].double().cpu().numpy()
    rg = comp_gpu.rank[lo:hi].cpu().numpy()
    eps = float(np.sqrt(cfg.eps2))
    worst = check_sigma(sg, ora.sigma, eps, [0, hi - lo], ora.rank)
    print(f"  unit ({s},{h}) sigma worst err/bound {worst:.3g}")
    n_swap = check_ranks(rg, ora.rank, ora.sigma, [0, hi - lo], [R])
    pool = s * cfg.n_kv_heads + h
    check_objective(obj_gpu[pool:pool + 1].cpu().numpy(), sg, rg, ora.objective, ora.sigma, ora.rank,
                    [0, hi - lo], cfg.eps2)
    # sampled reconstructions (first, middle, last block of the pool)
    picks = [0, (hi - lo) // 2, hi - lo - 1]
    ids = torch.tensor([lo + b for b in picks], dtype=torch.int32, device=DEV)
    xh = torch.empty((len(picks), cfg.block_len, cfg.head_dim), dtype=torch.float32, device=DEV)
    milo_reconstruct(comp_gpu, ids, xh)
    xh = xh.double().cpu().numpy()
    for i, b in enumerate(picks):
        r = int(rg[b])
        if r == int(ora.rank[b]):
            ref = oracle.reconstruct(ora.A[b], ora.B[b])
        else:
            A, B = oracle.project(X64[b], ora.V[b], r)
            ref = oracle.reconstruct(*oracle.store(A, B, storage))
        rel = np.linalg.norm(xh[i] - ref) / max(np.linalg.norm(ref), 1e-300)
        assert rel <= RECON_TOL[storage], f"unit ({s},{h}) block {b}: rel-F {rel:.3g}"
    print(f"  unit ({s},{h}) ranks {int(rg.min())}..{int(rg.max())}, rank swaps {n_swap}")
    return oracle.reconstruct_blocks(ora)


# attention tolerance (x max|v|) per factor storage, as in the small cases
ATT_TOL = {"bf16": 2e-2, "f32": 2e-2, "i4": 5e-2, "i2": 5e-2}


def _run_workload(cfg_idx, units, storage=None):
    cfg = CONFIGS[cfg_idx]
    st = storage or cfg.storage
    pp, bud = layer_pools(cfg)
    Xk = layer_inputs(cfg, 0, "k", device=DEV)
    Xv = layer_inputs(cfg, 0, "v", device=DEV)
    kf, sk, ok, _ = run_gpu_compress(Xk, pp, bud, cfg.eps2, st)
    vf, sv, ov, _ = run_gpu_compress(Xv, pp, bud, cfg.eps2, st)
    q = queries(cfg, 0, scale=Q_SCALE)
    q_pos = torch.full((cfg.batch,), cfg.context_len + cfg.tail_len, dtype=torch.int64)
    sel = selection(cfg)
    kw, tails = {}, None
    if sel is not None:
        kw.update(sel_ptr=torch.tensor(np.cumsum([0] + [len(x) for x in sel]), dtype=torch.int32, device=DEV),
                  sel_blk=torch.tensor(sum(sel, []), dtype=torch.int32, device=DEV), sel_max=cfg.sel_blocks)
    if cfg.tail_len:
        tails = (tail_inputs(cfg, 0, "k", device=DEV), tail_inputs(cfg, 0, "v", device=DEV))
        kw.update(tail_k=tails[0], tail_v=tails[1],
                  tail_len=torch.full((cfg.batch,), cfg.tail_len, dtype=torch.int32, device=DEV),
                  tail_pos0=torch.full((cfg.batch,), cfg.context_len, dtype=torch.int64, device=DEV))
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    milo_decode_attention(q.to(DEV), q_pos.to(DEV), kf, vf, cfg.blocks_per_seq, cfg.n_kv_heads, out, **kw)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    G = cfg.group
    for s, h in units:
        Kh = _check_unit(cfg, s, h, Xk, kf, sk, ok, st)
        Vh = _check_unit(cfg, s, h, Xv, vf, sv, ov, st)
        tkw = {}
        if tails is not None:
            tkw = dict(tail_k=tails[0][s:s + 1, h:h + 1].double().cpu().numpy(),
                       tail_v=tails[1][s:s + 1, h:h + 1].double().cpu().numpy(),
                       tail_len=[cfg.tail_len], tail_pos0=[cfg.context_len])
        ref = oracle.decode(q[s:s + 1, h * G:(h + 1) * G].double().numpy(), [int(q_pos[s])],
                            Kh, Vh, cfg.block_len, 1, cfg.blocks_per_seq,
                            sel=None if sel is None else [sel[s]], rope_base=cfg.rope_base, **tkw)
        err = np.abs(got[s, h * G:(h + 1) * G] - ref[0]).max()
        vmax = max(np.abs(Vh).max(), float(tails[1][s, h].abs().max()) if tails is not None else 0.0)
        print(f"  unit ({s},{h}) attention max|err| {err:.3g} max|ref| {np.abs(ref).max():.3g} "
              f"max|v| {vmax:.3g}")
        assert err <= ATT_TOL[st]
        assert err <= ATT_TOL[st] * vmax


def test_fullsize_long_context_layer():
    _run_workload(4, [(0, 0), (11, 1)])


def test_fullsize_selection_and_tail_layer():
    _run_workload(2, [(0, 0), (5, 3)])


@pytest.mark.parametrize("storage", ["i4", "i2"])
def test_fullsize_long_context_lowbit(storage):
    """The long-context layer with 4- or 2-bit factors: codes from the fp32-accurate
    factors, decoded in the benchmark's launch configuration."""
    _run_workload(4, [(7, 1)], storage=storage)
