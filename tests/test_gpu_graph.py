"""Decode attention recorded into a graph (torch.cuda.CUDAGraph over the C ABI
launches) and replayed: every replay must reproduce the eager result bit for
bit.  The replays are interleaved with eager decodes of other inputs into
other outputs and with synchronisations, and the graph's outputs are
overwritten before each replay, so a replay that wrote nothing or wrote stale
values would be seen."""
import numpy as np
import pytest
import torch

from block_wise_rank_amd import Factors, milo_decode_attention
from synthetic.factors import random_factor_set

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _factors(storage, n, T, seed, ranks):
    t, _, _ = random_factor_set(n, T, 128, storage, seed=seed, ranks=ranks)
    return Factors(storage, n, T, 128, rank=t["rank"].to(DEV), a_off=t["a_off"].to(DEV),
                   b_off=t["b_off"].to(DEV), arena=t["arena"].to(DEV))


@pytest.mark.parametrize("storage", ["bf16", "i4"])
def test_decode_graph_replays_match_eager(storage):
    batch, hkv, hq, T, bps, layers = 2, 2, 16, 1024, 4, 3
    n = batch * hkv * bps
    ranks = np.random.default_rng(3).integers(1, 129, size=n)
    kf = [_factors(storage, n, T, 100 + 2 * l, ranks) for l in range(layers)]
    vf = [_factors(storage, n, T, 101 + 2 * l, ranks[::-1].copy()) for l in range(layers)]
    g = torch.Generator().manual_seed(11)
    q = [(torch.randn((batch, hq, 128), generator=g) * 4).to(torch.bfloat16).to(DEV) for _ in range(layers)]
    q_pos = torch.tensor([bps * T, bps * T + 9], dtype=torch.int64, device=DEV)
    outs = [torch.empty((batch, hq, 128), dtype=torch.float32, device=DEV) for _ in range(layers)]

    def step(dst, queries):
        for l in range(layers):
            milo_decode_attention(queries[l], q_pos, kf[l], vf[l], bps, hkv, dst[l])

    eager = [torch.empty_like(o) for o in outs]
    step(eager, q)
    torch.cuda.synchronize()
    # warm the outputs of the graph once eagerly, then record
    step(outs, q)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(outs, q)
    other_q = [(qq.float() * -0.5).to(torch.bfloat16) for qq in q]
    other = [torch.empty_like(o) for o in outs]
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        step(other, other_q)  # eager work between replays
        torch.cuda.synchronize()
        for l in range(layers):
            assert torch.equal(outs[l], eager[l]), f"replay {rep}, layer {l}"
        assert not torch.equal(other[0], eager[0])
