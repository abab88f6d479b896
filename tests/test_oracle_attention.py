"""Pins for the oracle's RoPE and decode attention.

Keys are compressed before RoPE (evolve.pub review, Summary and Strengths; the
ai4snews Figure 1 caption speaks of pre-RoPE keys), so attention rotates the
rebuilt keys at their absolute positions.  Pins: RoPE against the independent
complex-exponential form, its norm and relative-position properties, attention
against torch's fp64 scaled-dot-product attention, and closed-form cases.
"""
import numpy as np
import pytest
import torch

BASE = 1e6


def _rope_complex(x, pos, base=BASE):
    """RoPE written as multiplication of z_j = x_j + i x_{j+d/2} by exp(i pos theta_j)."""
    d = x.shape[-1]
    h = d // 2
    theta = base ** (-2.0 * np.arange(h) / d)
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * np.multiply.outer(pos, theta))
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_matches_complex_form(oracle_lib):
    rng = np.random.default_rng(0)
    for pos in [0, 1, 7, 1000, 65791, 131071]:
        x = rng.standard_normal(128)
        got = oracle_lib.rope(x, pos, BASE)
        ref = _rope_complex(x, np.float64(pos))
        assert np.abs(got - ref).max() <= 1e-9


def test_rope_identity_and_norm(oracle_lib):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(128)
    assert np.array_equal(oracle_lib.rope(x, 0, BASE), x)
    y = oracle_lib.rope(x, 123457, BASE)
    assert abs(np.linalg.norm(y) - np.linalg.norm(x)) <= 1e-12 * np.linalg.norm(x)


def test_rope_relative_position(oracle_lib):
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    a, b = 70000, 3
    ref = oracle_lib.rope(q, a, BASE) @ oracle_lib.rope(k, b, BASE)
    for delta in [1, 513, 40000]:
        got = oracle_lib.rope(q, a + delta, BASE) @ oracle_lib.rope(k, b + delta, BASE)
        assert abs(got - ref) <= 1e-9 * (np.linalg.norm(q) * np.linalg.norm(k))


def test_attention_matches_torch_sdpa(oracle_lib):
    rng = np.random.default_rng(3)
    n, d = 300, 128
    q = rng.standard_normal(d) * 3
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    pos = np.sort(rng.choice(70000, size=n, replace=False))
    q_pos = 70001
    got = oracle_lib.attention(q, q_pos, K, V, pos, BASE, 1 / np.sqrt(d))
    qr = torch.from_numpy(_rope_complex(q, np.float64(q_pos)))[None, None, None]
    kr = torch.from_numpy(_rope_complex(K, pos.astype(np.float64)))[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qr, kr, torch.from_numpy(V)[None, None])
    assert np.abs(got - ref[0, 0, 0].numpy()).max() <= 1e-12


def test_attention_closed_forms(oracle_lib):
    rng = np.random.default_rng(4)
    d = 128
    K = rng.standard_normal((10, d))
    V = rng.standard_normal((10, d))
    pos = np.arange(10)
    # One token: the output is that token's value.
    out = oracle_lib.attention(rng.standard_normal(d), 11, K[:1], V[:1], pos[:1], BASE, 0.1)
    assert np.abs(out - V[0]).max() <= 1e-15
    # Zero query: every logit is 0 and the output is the mean of V.
    out = oracle_lib.attention(np.zeros(d), 11, K, V, pos, BASE, 0.1)
    assert np.abs(out - V.mean(axis=0)).max() <= 1e-14
    # Huge logits stay finite (the max is subtracted) and pick the arg-max token.
    q = K[3] * 1e4
    out = oracle_lib.attention(q, 0, K, V, np.zeros(10, dtype=np.int64), BASE, 1.0)
    assert np.all(np.isfinite(out)) and np.abs(out - V[3]).max() <= 1e-12


def test_decode_full_rank_equals_attention_on_raw_cache(oracle_lib):
    """With full-rank fp64 factors the compressed decode equals attention over the
    raw K/V: the whole oracle pipeline (SVD -> allocation -> factors -> decode)
    against the plain definition."""
    from synthetic import planted_blocks
    nb, T, d = 4, 128, 128
    Xk = planted_blocks(nb, T, d, (4.0, 24.0), 41, out_dtype="f64").numpy()
    Xv = planted_blocks(nb, T, d, (16.0, 64.0), 42, out_dtype="f64").numpy()
    ck = oracle_lib.compress(Xk, [0, nb], [nb * d], 1e-4, "f32")
    cv = oracle_lib.compress(Xv, [0, nb], [nb * d], 1e-4, "f32")
    assert (ck.rank == d).all() and (cv.rank == d).all()
    Kh = [oracle_lib.reconstruct(ck.A[b], ck.B[b]) for b in range(nb)]
    Vh = [oracle_lib.reconstruct(cv.A[b], cv.B[b]) for b in range(nb)]
    q = np.random.default_rng(5).standard_normal((1, 2, d)) * 20
    qpos = [nb * T]
    out = oracle_lib.decode(q, qpos, Kh, Vh, T, 1, nb)
    ref = oracle_lib.decode(q, qpos, list(Xk), list(Xv), T, 1, nb)
    # fp32 factor storage bounds the difference.
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(Xv).max()


def test_decode_selection_and_tail(oracle_lib):
    """Selected blocks keep their absolute positions; the tail follows the context."""
    rng = np.random.default_rng(6)
    T, d, nblk = 64, 128, 5
    K = [rng.standard_normal((T, d)) for _ in range(nblk)]
    V = [rng.standard_normal((T, d)) for _ in range(nblk)]
    tk = rng.standard_normal((1, 1, 16, d))
    tv = rng.standard_normal((1, 1, 16, d))
    q = rng.standard_normal((1, 1, d)) * 5
    sel = [[1, 3]]
    out = oracle_lib.decode(q, [nblk * T + 10], K, V, T, 1, nblk, sel=sel,
                            tail_k=tk, tail_v=tv, tail_len=[10], tail_pos0=[nblk * T])
    Kc = np.concatenate([K[1], K[3], tk[0, 0, :10]])
    Vc = np.concatenate([V[1], V[3], tv[0, 0, :10]])
    pos = np.concatenate([np.arange(T) + T, np.arange(T) + 3 * T, np.arange(10) + nblk * T])
    ref = oracle_lib.attention(q[0, 0], nblk * T + 10, Kc, Vc, pos, BASE, 1 / np.sqrt(d))
    assert np.abs(out[0, 0] - ref).max() <= 1e-15


def _sdpa_reference(q, q_pos, K_all, V_all, sel, block_len):
    """Decode by torch's fp64 attention with its own grouped-query mapping
    (enable_gqa: query head j of a group of G reads KV head j // G).  The cache
    is a [batch, Hkv, blocks, T, d] array; a sequence's attended blocks are
    sliced out of it and concatenated in order, so nothing here repeats the
    oracle's block-id arithmetic."""
    batch, Hq, d = q.shape
    out = np.zeros((batch, Hq, d))
    for s in range(batch):
        blocks = list(sel[s])
        Kc = K_all[s][:, blocks].reshape(K_all.shape[1], -1, d)   # [Hkv, L, d]
        Vc = V_all[s][:, blocks].reshape(V_all.shape[1], -1, d)
        pos = np.concatenate([np.arange(block_len) + b * block_len for b in blocks]).astype(np.float64)
        qr = torch.from_numpy(_rope_complex(q[s], np.float64(q_pos[s])))[None, :, None]   # [1, Hq, 1, d]
        kr = torch.from_numpy(_rope_complex(Kc, pos))[None]
        o = torch.nn.functional.scaled_dot_product_attention(qr, kr, torch.from_numpy(Vc)[None],
                                                             enable_gqa=True)
        out[s] = o[0, :, 0].numpy()
    return out


def test_decode_batches_kv_heads_and_groups(oracle_lib):
    """Several sequences, KV heads and query-head groups: the oracle's decode
    equals torch's grouped-query attention over the same cache laid out as
    [sequence, KV head, block, token, dim], with the factor block list in that
    order (block id = position in the flattened layout), per-sequence query
    positions and per-sequence block selections."""
    rng = np.random.default_rng(7)
    batch, Hkv, G, bps, T, d = 2, 2, 4, 3, 16, 128
    K_all = rng.standard_normal((batch, Hkv, bps, T, d))
    V_all = rng.standard_normal((batch, Hkv, bps, T, d))
    q = rng.standard_normal((batch, Hkv * G, d)) * 4
    q_pos = [bps * T, bps * T + 5]
    K_list = list(K_all.reshape(-1, T, d))
    V_list = list(V_all.reshape(-1, T, d))
    got = oracle_lib.decode(q, q_pos, K_list, V_list, T, Hkv, bps)
    ref = _sdpa_reference(q, q_pos, K_all, V_all, [range(bps)] * batch, T)
    assert np.abs(got - ref).max() <= 1e-12
    sel = [[0, 2], [1]]
    got = oracle_lib.decode(q, q_pos, K_list, V_list, T, Hkv, bps, sel=sel)
    ref = _sdpa_reference(q, q_pos, K_all, V_all, sel, T)
    assert np.abs(got - ref).max() <= 1e-12
