"""Host-offloaded compressed cache (milo_fetch_blocks): factor sets kept in
pinned host memory, the blocks a decode step attends brought to the device.

The fetch is pure data movement, so its parity is equality: the fetched bytes
equal the host bytes, blocks not listed are left untouched, and decode over the
fetched set is bit-identical to decode over a device-resident set; the decode
over the fetched set is also checked against the oracle's decode of the
decoded factor values the generator wrote (the same tolerances as the resident
decode tests).
"""
import numpy as np
import pytest
import torch

import oracle

from block_wise_rank_amd import Factors, MiloError, milo_decode_attention, milo_fetch_blocks
from synthetic.factors import i2_rank_bytes, i4_rank_bytes, random_factor_set

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _set(tensors, storage, n, T, device):
    f = Factors(storage, n, T, 128, rank=tensors["rank"].to(device), a_off=tensors["a_off"].to(device),
                b_off=tensors["b_off"].to(device), arena=tensors["arena"].to(device))
    if storage == "i8":
        f.a_scale = tensors["a_scale"].to(device)
        f.b_scale = tensors["b_scale"].to(device)
    return f


def _decode(q, q_pos, kf, vf, bps, hkv, sel_ptr, sel_blk, sel_max):
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    milo_decode_attention(q, q_pos, kf, vf, bps, hkv, out, sel_ptr=sel_ptr, sel_blk=sel_blk, sel_max=sel_max)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("storage", ["bf16", "i8", "i4", "i2", "f32"])
def test_fetch_then_decode_equals_resident(storage):
    batch, hkv, hq, T, bps = 2, 2, 16, 512, 8
    n = batch * hkv * bps
    ranks = np.random.default_rng(4).integers(0, 129, size=n)
    ranks[3] = 0
    kt, kA, kB = random_factor_set(n, T, 128, storage, seed=31, ranks=ranks)
    vt, vA, vB = random_factor_set(n, T, 128, storage, seed=32, ranks=ranks[::-1].copy())
    k_res, v_res = _set(kt, storage, n, T, DEV), _set(vt, storage, n, T, DEV)
    k_host, v_host = k_res.to_host(), v_res.to_host()
    assert k_host.arena.is_pinned() and k_host.rank.device.type == "cpu"
    k_dev, v_dev = k_host.like(DEV), v_host.like(DEV)
    for f in (k_dev, v_dev):  # a pattern that must survive where nothing is fetched
        f.arena.fill_(0x5A)
        if f.a_scale is not None:
            f.a_scale.fill_(7.0)
            f.b_scale.fill_(7.0)
    # per sequence: blocks attended (ascending and distinct, as decode requires);
    # the fetch list names them in a scrambled order with repeats
    sel = [[0, 1, 2, 5], [3, 4, 7]]
    ids = sorted({(s * hkv + h) * bps + b for s in range(batch) for h in range(hkv) for b in sel[s]})
    listed = ids[::-1] + ids[:3]
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        milo_fetch_blocks(k_host, k_dev, listed, stream=st)
        milo_fetch_blocks(v_host, v_dev, listed, stream=st)
    st.synchronize()

    if storage == "i4":
        abpr, bbpr = i4_rank_bytes(T, 128)
    elif storage == "i2":
        abpr, bbpr = i2_rank_bytes(T, 128)
    else:
        e = {"f32": 4, "bf16": 2, "i8": 1}[storage]
        abpr, bbpr = T * e, 128 * e
    for host, dev in ((k_host, k_dev), (v_host, v_dev)):
        arena_h, arena_d = host.arena, dev.arena.cpu()
        touched = np.zeros(arena_h.numel(), dtype=bool)
        for b in ids:
            r = int(host.rank[b])
            for off, ln in ((int(host.a_off[b]), r * abpr), (int(host.b_off[b]), r * bbpr)):
                assert torch.equal(arena_d[off:off + ln], arena_h[off:off + ln]), f"block {b}"
                touched[off:off + ln] = True
        assert bool((arena_d.numpy()[~touched] == 0x5A).all()), "bytes outside the listed blocks changed"
        if storage == "i8":
            for b in ids:
                assert torch.equal(dev.a_scale.cpu()[b * T:(b + 1) * T], host.a_scale[b * T:(b + 1) * T])
            assert float(dev.a_scale.cpu()[[b * T for b in range(n) if b not in ids]].min()) == 7.0

    sel_ptr = torch.tensor(np.cumsum([0] + [len(x) for x in sel]), dtype=torch.int32, device=DEV)
    sel_blk = torch.tensor(sum(sel, []), dtype=torch.int32, device=DEV)
    g = torch.Generator().manual_seed(2)
    q = (torch.randn((batch, hq, 128), generator=g) * 3).to(torch.float32 if storage == "f32" else torch.bfloat16)
    q = q.to(DEV)
    q_pos = torch.tensor([bps * T, bps * T + 9], dtype=torch.int64, device=DEV)
    want = _decode(q, q_pos, k_res, v_res, bps, hkv, sel_ptr, sel_blk, 4)
    got = _decode(q, q_pos, k_dev, v_dev, bps, hkv, sel_ptr, sel_blk, 4)
    assert torch.equal(got, want), f"max diff {float((got - want).abs().max())}"
    # the decode over the fetched set against the oracle on the decoded factors
    Kh = [a @ b for a, b in zip(kA, kB)]
    Vh = [a @ b for a, b in zip(vA, vB)]
    ref = oracle.decode(q.to(torch.float64).cpu().numpy(), q_pos.cpu().numpy(), Kh, Vh, T, hkv, bps, sel=sel)
    vmax = max(float(np.abs(Vh[(s * hkv + h) * bps + b]).max()) for s in range(batch) for h in range(hkv)
               for b in sel[s])
    err = float(np.abs(got.cpu().numpy() - ref).max())
    tol = {"bf16": 2e-2, "i8": 2e-2, "i4": 5e-2, "i2": 5e-2, "f32": 1e-4}[storage]
    print(f"\n[offload {storage}] max|err| vs oracle {err:.3g}, bound {tol * vmax:.3g}")
    assert err <= tol * vmax


def test_fetch_rejects_bad_ids_and_geometry():
    n, T = 4, 256
    kt, _, _ = random_factor_set(n, T, 128, "bf16", seed=1)
    res = _set(kt, "bf16", n, T, DEV)
    host = res.to_host()
    dev = host.like(DEV)
    with pytest.raises(MiloError):
        milo_fetch_blocks(host, dev, [0, 4])
    with pytest.raises(MiloError):
        milo_fetch_blocks(host, dev, [-1])
    small = Factors.alloc("bf16", n, T, 128, 256, device=DEV)
    with pytest.raises(MiloError):
        milo_fetch_blocks(host, small, [0])
    with pytest.raises(ValueError):
        milo_fetch_blocks(res, dev, [0])  # a device-resident source is not an offloaded set
    milo_fetch_blocks(host, dev, [])      # nothing to do
