"""Pins for the oracle's factors (A = X V_r, B = V_r^T), reconstruction and
storage encodings.

The pages say the cache is stored per block in low-rank form and only the needed
blocks are rebuilt (evolve.pub review, FAQ).  Pins: identity at full rank, the
Eckart-Young identity and optimality (against LAPACK's truncated SVD), and the
encodings against hand-computed values and torch's fp32 -> bf16 conversion.
"""
import numpy as np
import pytest
import torch

from synthetic import planted_blocks


@pytest.fixture(scope="module")
def block(oracle_lib):
    X = planted_blocks(1, 256, 128, (4.0, 32.0), 31, out_dtype="f64").numpy()[0]
    sigma, V, _ = oracle_lib.svd_blocks(X[None])
    return X, sigma[0], V[0]


def test_identity_at_full_rank(oracle_lib, block):
    X, sigma, V = block
    A, B = oracle_lib.project(X, V, 128)
    assert np.abs(oracle_lib.reconstruct(A, B) - X).max() <= 1e-12


def test_zero_rank(oracle_lib, block):
    X, sigma, V = block
    A, B = oracle_lib.project(X, V, 0)
    assert A.shape == (256, 0) and B.shape == (0, 128)
    assert (oracle_lib.reconstruct(A, B) == 0).all()


@pytest.mark.parametrize("r", [1, 7, 40, 64, 127])
def test_eckart_young(oracle_lib, block, r):
    X, sigma, V = block
    A, B = oracle_lib.project(X, V, r)
    Xh = oracle_lib.reconstruct(A, B)
    err2 = np.sum((X - Xh) ** 2)
    tail = np.sum(sigma[r:] ** 2)
    assert abs(err2 - tail) <= 1e-12 * np.sum(sigma ** 2)
    # Same error as LAPACK's best rank-r approximation.
    U, S, Vt = np.linalg.svd(X, full_matrices=False)
    best = (U[:, :r] * S[:r]) @ Vt[:r]
    assert abs(np.sum((X - best) ** 2) - err2) <= 1e-12 * np.sum(sigma ** 2)
    # B has orthonormal rows, A = X B^T.
    assert np.abs(B @ B.T - np.eye(r)).max() <= 1e-13
    assert np.abs(A - X @ B.T).max() <= 1e-12


def test_round_bf16_hand_values(oracle_lib):
    e = 2.0 ** -8
    cases = {
        1.0: 1.0,
        1.0 + e: 1.0,                       # halfway, ties to the even mantissa
        1.0 + 3 * e: 1.0 + 4 * e,           # halfway, rounds up to even
        1.0 + 1.5 * e: 1.0 + 2 * e,         # above halfway
        -(1.0 + e): -1.0,
        2.0 ** -133: 2.0 ** -133,           # smallest subnormal
        2.0 ** -134: 0.0,                   # halfway to zero, ties to even
        1.5 * 2.0 ** -134: 2.0 ** -133,
        3.0e38: 226.0 * 2.0 ** 120,         # 3.0e38 / 2^120 = 225.69
        3.5e38: np.inf,
        0.0: 0.0,
    }
    xs = np.array(list(cases.keys()))
    got = oracle_lib.round_bf16(xs)
    assert np.array_equal(got, np.array(list(cases.values())))


def test_round_bf16_matches_torch_on_fp32_values(oracle_lib):
    """For inputs already exact in fp32, rounding fp64 -> bf16 directly equals
    torch's fp32 -> bf16 conversion (a single rounding either way)."""
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 8)).float()
    ref = x.to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle_lib.round_bf16(x.to(torch.float64).numpy())
    assert np.array_equal(got, ref)


def test_round_bf16_is_a_single_rounding(oracle_lib):
    """A value just above a bf16 halfway point that fp32 would round onto the
    halfway point: single rounding from fp64 must round up."""
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert oracle_lib.round_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7


def test_round_f32(oracle_lib):
    x = np.random.default_rng(1).standard_normal(1000)
    assert np.array_equal(oracle_lib.round_f32(x), x.astype(np.float32).astype(np.float64))


def test_int8_hand_values(oracle_lib):
    M = np.array([[127.0, -63.5, 0.5, 0.0],
                  [254.0, 1.0, 3.0, -254.0],
                  [0.0, 0.0, 0.0, 0.0],
                  [-10.0, 2.5, 7.5, 1.0]])
    scale, codes, deq = oracle_lib.quant_int8_rows(M)
    assert scale[0] == 1.0 and list(codes[0]) == [127, -64, 0, 0]
    assert scale[1] == 2.0 and list(codes[1]) == [127, 0, 2, -127]
    assert scale[2] == 0.0 and list(codes[2]) == [0, 0, 0, 0] and (deq[2] == 0).all()
    s3 = np.float32(10.0) / np.float32(127.0)
    assert scale[3] == float(s3)
    assert codes[3][0] == -127
    assert list(codes[3][1:]) == [int(np.rint(np.float32(v) / s3)) for v in (2.5, 7.5, 1.0)]


def test_int8_error_bound(oracle_lib):
    rng = np.random.default_rng(4)
    M = rng.standard_normal((64, 96)) * np.exp(rng.standard_normal((64, 1)))
    scale, codes, deq = oracle_lib.quant_int8_rows(M)
    assert (np.abs(codes.astype(int)) <= 127).all()
    assert (np.abs(codes).max(axis=1) == 127).all()
    # |x - q s| <= s/2 plus the fp32 rounding of x and of s.
    bound = scale[:, None] * (0.5 + 1e-5) + np.abs(M) * 2e-7
    assert (np.abs(deq - M) <= bound).all()


def test_int4_hand_values(oracle_lib):
    """Groups of 4 for hand values (the group length is a parameter): s = max|x|/7,
    codes rint(x/s) with ties to even, each group on its own."""
    M = np.array([[7.0, -3.5, 0.5, 0.0, 14.0, 1.0, 3.0, -14.0],
                  [0.0, 0.0, 0.0, 0.0, -1.0, 0.25, 0.5, 0.0]])
    scale, codes, deq = oracle_lib.quant_int4_groups(M, group=4)
    assert scale[0].tolist() == [1.0, 2.0]
    assert list(codes[0]) == [7, -4, 0, 0, 7, 0, 2, -7]
    assert scale[1][0] == 0.0 and list(codes[1][:4]) == [0, 0, 0, 0] and (deq[1][:4] == 0).all()
    s = np.float32(1.0) / np.float32(7.0)
    assert scale[1][1] == float(s)
    assert list(codes[1][4:]) == [-7] + [int(np.rint(np.float32(v) / s)) for v in (0.25, 0.5, 0.0)]
    assert deq[0][1] == -4.0 and deq[0][6] == 4.0


def test_int4_error_bound_and_groups(oracle_lib):
    rng = np.random.default_rng(5)
    M = rng.standard_normal((48, 256)) * np.exp(2 * rng.standard_normal((48, 8))).repeat(32, axis=1)
    scale, codes, deq = oracle_lib.quant_int4_groups(M)
    assert scale.shape == (48, 8)
    assert (np.abs(codes.astype(int)) <= 7).all()
    # every group reaches +-7 at its largest element
    assert (np.abs(codes.reshape(48, 8, 32)).max(axis=2) == 7).all()
    # |x - q s| <= s/2 plus the fp32 rounding of x and of s
    bound = np.repeat(scale, 32, axis=1) * (0.5 + 1e-5) + np.abs(M) * 2e-7
    assert (np.abs(deq - M) <= bound).all()
    # groups are independent: changing one group changes nothing else
    M2 = M.copy()
    M2[3, 64:96] *= 100.0
    s2, c2, _ = oracle_lib.quant_int4_groups(M2)
    keep = np.ones((48, 8), dtype=bool)
    keep[3, 2] = False
    assert np.array_equal(s2[keep], scale[keep])
    assert np.array_equal(c2.reshape(48, 8, 32)[keep], codes.reshape(48, 8, 32)[keep])
    # the dequantised values quantise to themselves
    s3, c3, d3 = oracle_lib.quant_int4_groups(deq)
    assert np.array_equal(c3, codes) and np.allclose(d3, deq, rtol=1e-6, atol=0)


def test_int2_hand_values(oracle_lib):
    """Groups of 4 for hand values: s = max|x|/3, code c for the nearest level
    (2c - 3) s, |x|/s = 2 going to the outer level, 0 to +s, a zero run to code 2."""
    M = np.array([[3.0, -1.0, 2.0, -2.0, 6.0, 0.0, -1.5, 1.0],
                  [0.0, 0.0, 0.0, 0.0, -0.3, 0.1, 0.25, -0.19]])
    scale, codes, deq = oracle_lib.quant_int2_groups(M, group=4)
    assert scale[0].tolist() == [1.0, 2.0]
    assert list(codes[0]) == [3, 1, 3, 0, 3, 2, 1, 2]
    assert deq[0].tolist() == [3.0, -1.0, 3.0, -3.0, 6.0, 2.0, -2.0, 2.0]
    assert scale[1][0] == 0.0 and list(codes[1][:4]) == [2, 2, 2, 2] and (deq[1][:4] == 0).all()
    s = np.float32(np.float32(0.3) / np.float32(3.0))
    assert scale[1][1] == float(s)
    assert list(codes[1][4:]) == [0, 2, 3, 1]
    assert deq[1][4:].tolist() == [float(np.float32(k) * s) for k in (-3, 1, 3, -1)]


def test_int2_error_bound_and_groups(oracle_lib):
    rng = np.random.default_rng(6)
    M = rng.standard_normal((48, 256)) * np.exp(2 * rng.standard_normal((48, 8))).repeat(32, axis=1)
    scale, codes, deq = oracle_lib.quant_int2_groups(M)
    assert scale.shape == (48, 8) and codes.max() <= 3
    # the largest element of every group lands on an outer level, +-3 s
    g = M.reshape(48, 8, 32)
    top = np.abs(g).argmax(axis=2)
    ctop = np.take_along_axis(codes.reshape(48, 8, 32), top[..., None], axis=2)[..., 0]
    assert np.array_equal(ctop, np.where(np.take_along_axis(g, top[..., None], axis=2)[..., 0] < 0, 0, 3))
    # levels 2s apart, the outer ones at +-max: |x - x~| <= s plus fp32 rounding
    bound = np.repeat(scale, 32, axis=1) * (1 + 1e-5) + np.abs(M) * 2e-7
    assert (np.abs(deq - M) <= bound).all()
    # the dequantised value has the sign of x
    assert (np.sign(deq) == np.where(M < 0, -1, 1)).all()
    M2 = M.copy()
    M2[5, 160:192] *= -100.0
    s2, c2, _ = oracle_lib.quant_int2_groups(M2)
    keep = np.ones((48, 8), dtype=bool)
    keep[5, 5] = False
    assert np.array_equal(s2[keep], scale[keep])
    assert np.array_equal(c2.reshape(48, 8, 32)[keep], codes.reshape(48, 8, 32)[keep])
    # the dequantised values quantise to themselves
    s3, c3, d3 = oracle_lib.quant_int2_groups(deq)
    assert np.array_equal(c3, codes) and np.allclose(d3, deq, rtol=1e-6, atol=0)


def test_int2_decision_without_division():
    """The 2-bit decision fl(|x| / s) >= 2 (fp32, correctly rounded) equals
    |x| >= 2 s for every fp32 x and s > 0: the projection kernel takes it that
    way.  Checked on random scales over many binades, at 2 s and its fp32
    neighbours, and on random values."""
    rng = np.random.default_rng(7)
    s = (rng.uniform(1, 2, 20000) * 2.0 ** rng.integers(-140, 120, 20000)).astype(np.float32)
    s = np.concatenate([s, np.float32(2.0) ** np.arange(-149, 127).astype(np.float32)])
    two_s = (np.float32(2) * s).astype(np.float32)
    xs = [two_s, np.nextafter(two_s, np.float32(0)), np.nextafter(two_s, np.float32(np.inf)),
          (s * rng.uniform(0, 3, s.size)).astype(np.float32)]
    with np.errstate(all="ignore"):
        for x in xs:
            ok = np.isfinite(x) & (s > 0)
            q = (x[ok] / s[ok]).astype(np.float32)
            assert np.array_equal(q >= np.float32(2), x[ok] >= two_s[ok])


def test_store_roundtrip_shapes(oracle_lib, block):
    X, sigma, V = block
    A, B = oracle_lib.project(X, V, 50)
    for st in ("f32", "bf16", "i8", "i4", "i2"):
        As, Bs = oracle_lib.store(A, B, st)
        assert As.shape == A.shape and Bs.shape == B.shape
        rel = np.linalg.norm(oracle_lib.reconstruct(As, Bs) - oracle_lib.reconstruct(A, B)) / \
            np.linalg.norm(oracle_lib.reconstruct(A, B))
        # 4-bit: each element moves by at most s/2 = max|group|/14; 2-bit: by at
        # most s = max|group|/3
        assert rel <= {"f32": 1e-6, "bf16": 1e-2, "i8": 3e-2, "i4": 0.2, "i2": 0.8}[st]
