"""milo_decode_attention_noalloc: the decode entry point for callers that cannot
allocate, using the library's static per-GPU scratch.  It runs the same kernels
as milo_decode_attention, so on the same inputs its output must equal that
entry point's bit for bit; two calls in a row (the second smaller, so it reads
a scratch the first call left behind) and a call that needs more scratch than
the static array holds (refused before anything is enqueued)."""
import numpy as np
import pytest
import torch

from block_wise_rank_amd import (Factors, MiloError, milo_decode_attention, milo_decode_attention_noalloc)
from synthetic.factors import random_factor_set

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _set(t, storage, n, T):
    f = Factors(storage, n, T, 128, rank=t["rank"].to(DEV), a_off=t["a_off"].to(DEV),
                b_off=t["b_off"].to(DEV), arena=t["arena"].to(DEV))
    if storage == "i8":
        f.a_scale, f.b_scale = t["a_scale"].to(DEV), t["b_scale"].to(DEV)
    return f


def _case(batch, hkv, G, T, bps, seed, storage="bf16", tail=0, rank_range=(0, 128)):
    n = batch * hkv * bps
    kt, _, _ = random_factor_set(n, T, 128, storage, seed=seed, rank_range=rank_range)
    vt, _, _ = random_factor_set(n, T, 128, storage, seed=seed + 1, rank_range=rank_range)
    kf, vf = _set(kt, storage, n, T), _set(vt, storage, n, T)
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn((batch, hkv * G, 128), generator=g) * 3).to(torch.bfloat16).to(DEV)
    q_pos = torch.arange(batch, dtype=torch.int64).add(bps * T + tail).to(DEV)
    kw = {}
    if tail:
        cap = 64 * ((tail + 63) // 64)
        kw = dict(tail_k=(torch.randn((batch, hkv, cap, 128), generator=g) * 0.3).to(torch.bfloat16).to(DEV),
                  tail_v=torch.randn((batch, hkv, cap, 128), generator=g).to(torch.bfloat16).to(DEV),
                  tail_len=torch.full((batch,), tail, dtype=torch.int32, device=DEV),
                  tail_pos0=torch.full((batch,), bps * T, dtype=torch.int64, device=DEV))
    return q, q_pos, kf, vf, bps, hkv, kw


def test_noalloc_equals_workspace_decode_twice():
    big = _case(4, 2, 8, 2048, 8, seed=100, tail=200)
    small = _case(1, 1, 4, 512, 3, seed=200, storage="i8")
    for q, q_pos, kf, vf, bps, hkv, kw in (big, small):
        want = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        milo_decode_attention(q, q_pos, kf, vf, bps, hkv, want, **kw)
        got = torch.full(q.shape, 7.0, dtype=torch.float32, device=DEV)
        milo_decode_attention_noalloc(q, q_pos, kf, vf, bps, hkv, got, **kw)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(got).all())
        assert torch.equal(got, want), float((got - want).abs().max())


def test_noalloc_refuses_calls_beyond_its_scratch():
    # 16 blocks x 8 splits of 128 tokens per (sequence, KV head), 16 sequences, 2 KV
    # heads, 16 query heads each: 65536 partials of 520 bytes, past the 32 MiB
    q, q_pos, kf, vf, bps, hkv, kw = _case(16, 2, 16, 1024, 16, seed=300, rank_range=(0, 4))
    out = torch.full(q.shape, 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(MiloError) as ei:
        milo_decode_attention_noalloc(q, q_pos, kf, vf, bps, hkv, out, split_len=128)
    torch.cuda.synchronize()
    assert "MILO_E_WORKSPACE" in str(ei.value)
    assert bool((out == 7.0).all())
