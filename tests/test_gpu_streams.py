"""Calls enqueued on a side stream with the scratch the binding allocates.

The library launches on the stream it is given; when the caller passes no
workspace the binding allocates it, and drops it when the call returns, while
the kernels may still be running on that stream.  The scratch is allocated with
the call's stream current, so torch's caching allocator cannot hand its memory
to work on another stream in the meantime.  Here the current stream overwrites
freshly allocated memory right after each call; the side-stream results must
equal those of the same calls on the current stream.
"""
import numpy as np
import pytest
import torch

from block_wise_rank_amd import Factors, milo_arena_bytes, milo_compress_blocks, milo_decode_attention
from synthetic import CONFIGS, layer_inputs, queries
from _parity import layer_pools

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _compress(X, pp, bud, cfg, stream=None):
    n, T, d = X.shape
    f = Factors.alloc("bf16", n, T, d, milo_arena_bytes("bf16", T, d, pp, bud), device=DEV)
    sigma = torch.zeros((n, d), dtype=torch.float32, device=DEV)
    milo_compress_blocks(X, pp, bud, cfg.eps2, sigma, f, stream=stream)
    return f, sigma


def test_side_stream_scratch_is_not_reused_by_other_streams():
    cfg = CONFIGS[1]
    pp, bud = layer_pools(cfg)
    Xk = layer_inputs(cfg, 0, "k", device=DEV)
    Xv = layer_inputs(cfg, 0, "v", device=DEV)
    kf0, s0 = _compress(Xk, pp, bud, cfg)
    vf0, _ = _compress(Xv, pp, bud, cfg)
    q = queries(cfg, 0, scale=300.0).to(DEV)
    q_pos = torch.full((cfg.batch,), cfg.context_len, dtype=torch.int64, device=DEV)
    out0 = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    milo_decode_attention(q, q_pos, kf0, vf0, cfg.blocks_per_seq, cfg.n_kv_heads, out0)
    torch.cuda.synchronize()
    ws_bytes = 64 << 20

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    kf1, s1 = _compress(Xk, pp, bud, cfg, stream=side)
    junk = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)  # current stream, right away
    junk.fill_(0xFF)
    vf1, _ = _compress(Xv, pp, bud, cfg, stream=side)
    junk2 = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    junk2.fill_(0x7F)
    out1 = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    milo_decode_attention(q, q_pos, kf1, vf1, cfg.blocks_per_seq, cfg.n_kv_heads, out1, stream=side)
    junk3 = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    junk3.fill_(0x3F)
    torch.cuda.synchronize()
    assert torch.equal(s1, s0)
    assert torch.equal(kf1.rank, kf0.rank) and torch.equal(kf1.arena, kf0.arena)
    assert torch.equal(vf1.arena, vf0.arena)
    assert torch.equal(out1, out0)
    del junk, junk2, junk3
