"""The C ABI without a GPU: the library loads, exports every symbol include/milo.h
declares, and rejects invalid arguments on the host before any HIP call."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from block_wise_rank_amd import _capi
    return _capi.load()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "milo.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(milo_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    from block_wise_rank_amd import _capi
    declared = _declared_functions()
    assert len(declared) >= 9
    for name in declared:
        assert hasattr(L, name), f"{name} declared in milo.h but not exported"
        assert name in _capi.SIGNATURES, f"{name} has no ctypes signature in the binding"


def test_versions_and_strings(L):
    assert L.milo_abi_version() == 4
    assert L.milo_status_string(0) == b"MILO_OK"
    assert L.milo_status_string(3) == b"MILO_E_WORKSPACE"


def _arr(typ, vals):
    return (typ * len(vals))(*vals)


def test_arena_bytes_formula_i4(L):
    """4-bit: per rank T/2 + T/8 bytes of A (codes, fp32 scales per 32 tokens)
    and d/2 + d/8 bytes of B."""
    pp = _arr(ctypes.c_int32, [0, 8, 8, 20])
    bud = _arr(ctypes.c_int64, [512, 5, 10 ** 6])
    n = L.milo_arena_bytes(3, 256, 128, ctypes.cast(pp, ctypes.c_void_p), 3,
                           ctypes.cast(bud, ctypes.c_void_p))
    assert n == (512 + 0 + 12 * 128) * ((128 + 32) + (64 + 16))


def test_arena_bytes_formula_i2(L):
    """2-bit: per rank T/4 + T/8 bytes of A (codes, fp32 scales per 32 tokens)
    and d/4 + d/8 bytes of B."""
    pp = _arr(ctypes.c_int32, [0, 8, 8, 20])
    bud = _arr(ctypes.c_int64, [512, 5, 10 ** 6])
    n = L.milo_arena_bytes(4, 256, 128, ctypes.cast(pp, ctypes.c_void_p), 3,
                           ctypes.cast(bud, ctypes.c_void_p))
    assert n == (512 + 0 + 12 * 128) * ((64 + 32) + (32 + 16))


def test_arena_bytes_formula(L):
    pp = _arr(ctypes.c_int32, [0, 8, 8, 20])
    bud = _arr(ctypes.c_int64, [512, 5, 10 ** 6])
    n = L.milo_arena_bytes(1, 256, 128, ctypes.cast(pp, ctypes.c_void_p), 3,
                           ctypes.cast(bud, ctypes.c_void_p))
    # pool 0: 512 ranks; pool 1 is empty; pool 2 is capped at 12 blocks x 128 ranks
    assert n == (512 + 0 + 12 * 128) * (256 + 128) * 2
    n8 = L.milo_arena_bytes(2, 256, 128, ctypes.cast(pp, ctypes.c_void_p), 3,
                            ctypes.cast(bud, ctypes.c_void_p))
    assert n8 * 2 == n


def test_memory_example_from_the_pages(L):
    """The worked example of the pages: an ~8 GB cache at 128K tokens becomes ~4 GB."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "memory_example.json")))
    T, d, L_, H = g["block_len"], g["head_dim"], g["layers"], g["n_kv_heads"]
    blocks = g["context_tokens"] // T
    R = int(g["budget_frac"] * blocks * d)
    n_pools = 2 * L_ * H  # K and V pools of every layer and KV head
    pp = _arr(ctypes.c_int32, [p * blocks for p in range(n_pools + 1)])
    bud = _arr(ctypes.c_int64, [R] * n_pools)
    compressed = L.milo_arena_bytes(1, T, d, ctypes.cast(pp, ctypes.c_void_p), n_pools,
                                    ctypes.cast(bud, ctypes.c_void_p))
    full = 2 * L_ * H * g["context_tokens"] * d * 2
    tol = g["relative_tolerance"]
    assert abs(full / 1e9 - g["full_cache_gb_stated"]) <= tol * g["full_cache_gb_stated"]
    assert abs(compressed / 1e9 - g["compressed_gb_stated"]) <= tol * g["compressed_gb_stated"]
    assert compressed / full == pytest.approx(0.5 * (1 + d / T))


def _blocks(x=0x1000, dtype=1, n=8, T=256, d=128, stride=128):
    from block_wise_rank_amd import _capi
    return _capi.milo_blocks(x, dtype, None, stride, n, T, d)


def _factors(dtype=1, n=8, T=256, d=128, arena=0x100000, nbytes=1 << 30):
    from block_wise_rank_amd import _capi
    return _capi.milo_factors(dtype, n, T, d, 0x2000, 0x3000, 0x4000, arena, nbytes, 0x5000,
                              0x6000)


def _compress(L, blocks, factors, pp=(0, 8), bud=(512,), eps2=1e-4, ws=None, wsb=0):
    ppa = _arr(ctypes.c_int32, list(pp))
    bda = _arr(ctypes.c_int64, list(bud))
    size = ctypes.c_size_t(wsb)
    st = L.milo_compress_blocks(ctypes.byref(blocks), ctypes.cast(ppa, ctypes.c_void_p),
                                len(pp) - 1, ctypes.cast(bda, ctypes.c_void_p), eps2, 0x7000,
                                None, ctypes.byref(factors), None, ws, ctypes.byref(size), None)
    return st, size.value


@pytest.mark.parametrize("case,expect", [
    ("head_dim", 2), ("block_len", 2), ("block_len_small", 2), ("in_dtype", 2), ("pair", 2),
    ("i4_block_len", 2), ("i2_block_len", 2),
    ("pool0", 1), ("pool_end", 1), ("pool_order", 1), ("budget_neg", 1), ("eps", 1),
    ("stride", 1), ("align", 1), ("geometry", 1), ("arena_small", 1), ("i8_scales", 1),
])
def test_compress_validation(L, case, expect):
    from block_wise_rank_amd import _capi
    b, f = _blocks(), _factors()
    kw = {}
    if case == "head_dim":
        b.head_dim = 64
    elif case == "block_len":
        b.block_len = 200
    elif case == "block_len_small":
        b.block_len = 64
    elif case == "in_dtype":
        b.dtype = 2
    elif case == "pair":
        f.dtype = 9  # no such factor dtype
    elif case == "i4_block_len":
        b.block_len = f.block_len = 192  # 4-bit factors need whole 128-token multiples
        f.dtype = 3
    elif case == "i2_block_len":
        b.block_len = f.block_len = 192  # so do 2-bit factors
        f.dtype = 4
    elif case == "pool0":
        kw["pp"] = (1, 8)
    elif case == "pool_end":
        kw["pp"] = (0, 7)
    elif case == "pool_order":
        kw["pp"], kw["bud"] = (0, 5, 3, 8), (1, 1, 1)
    elif case == "budget_neg":
        kw["bud"] = (-1,)
    elif case == "eps":
        kw["eps2"] = 0.0
    elif case == "stride":
        b.row_stride = 100
    elif case == "align":
        b.x = 0x1002
    elif case == "geometry":
        f.block_len = 512
    elif case == "arena_small":
        f.arena_bytes = 1000
    elif case == "i8_scales":
        f.dtype = 2
        f.a_scale = None
    st, _ = _compress(L, b, f, **kw)
    assert st == expect, L.milo_last_error()
    assert L.milo_last_error()


def test_compress_workspace_size_query(L):
    st, size = _compress(L, _blocks(), _factors())
    assert st == 3
    assert size >= 8 * 2 * 128 * 128 * 4
    assert size == L.milo_compress_workspace_bytes(8, 256, 128) - 0 or size > 0


def test_allocate_validation(L):
    pp = _arr(ctypes.c_int32, [0, 4])
    bud = _arr(ctypes.c_int64, [10])
    size = ctypes.c_size_t(0)
    args = lambda mr, n: (0x1000, n, 128, mr, ctypes.cast(pp, ctypes.c_void_p), 1,
                          ctypes.cast(bud, ctypes.c_void_p), 1e-4, 0x2000, None, None,
                          ctypes.byref(size), None)
    assert L.milo_allocate_ranks(*args(0, 4)) == 1
    assert L.milo_allocate_ranks(*args(129, 4)) == 1
    assert L.milo_allocate_ranks(*args(128, 3)) == 1     # CSR end != n_blocks
    assert L.milo_allocate_ranks(*args(128, 4)) == 3     # workspace size query
    assert size.value > 0


def test_unknown_allocation_policy_is_rejected(L):
    """The policy is validated before anything else, on the host."""
    from block_wise_rank_amd import _capi
    opts = _capi.milo_alloc_options(7, 0)
    pp = (ctypes.c_int32 * 2)(0, 4)
    bb = (ctypes.c_int64 * 1)(8)
    size = ctypes.c_size_t(0)
    st = L.milo_allocate_ranks_ex(0x1000, 4, 128, 128, ctypes.cast(pp, ctypes.c_void_p), 1,
                                  ctypes.cast(bb, ctypes.c_void_p), 1e-4, 0x2000, None,
                                  ctypes.byref(opts), None, ctypes.byref(size), None)
    assert st == _capi.MILO_E_INVALID and b"policy" in L.milo_last_error()
    blocks, f = _blocks(), _factors()
    st = L.milo_compress_blocks_ex(ctypes.byref(blocks), ctypes.cast(pp, ctypes.c_void_p), 1,
                                   ctypes.cast(bb, ctypes.c_void_p), 1e-4, 0x3000, None,
                                   ctypes.byref(f), None, ctypes.byref(opts), None,
                                   ctypes.byref(size), None)
    assert st == _capi.MILO_E_INVALID and b"policy" in L.milo_last_error()
    # a known policy passes this check and reaches the workspace size query
    ok = _capi.milo_alloc_options(_capi.MILO_ALLOC_RANDOM, 5)
    st = L.milo_allocate_ranks_ex(0x1000, 4, 128, 128, ctypes.cast(pp, ctypes.c_void_p), 1,
                                  ctypes.cast(bb, ctypes.c_void_p), 1e-4, 0x2000, None,
                                  ctypes.byref(ok), None, ctypes.byref(size), None)
    assert st == _capi.MILO_E_WORKSPACE and size.value > 0


def test_reconstruct_validation(L):
    f = _factors()
    assert L.milo_reconstruct(ctypes.byref(f), 0x10, 1, 0x20, 2, None) == 2   # int8 output
    assert L.milo_reconstruct(ctypes.byref(f), 0x10, -1, 0x20, 0, None) == 1
    assert L.milo_reconstruct(ctypes.byref(f), 0x10, 0, 0x20, 0, None) == 0   # nothing to do
    f.head_dim = 64
    assert L.milo_reconstruct(ctypes.byref(f), 0x10, 1, 0x20, 0, None) == 2


def _host_set(n=4, T=256, d=128, ranks=(8, 0, 128, 5), dtype=1):
    """A factor set whose metadata are host arrays (milo_fetch_blocks reads them
    on the host and rejects bad inputs before any HIP call)."""
    from block_wise_rank_amd import _capi
    rk = (ctypes.c_int32 * n)(*ranks)
    e = 2 if dtype == 1 else (4 if dtype == 0 else 1)
    sizes = [r * (T + d) * e for r in ranks]
    ao = [sum(sizes[:i]) for i in range(n)]
    bo = [ao[i] + ranks[i] * T * e for i in range(n)]
    aoff = (ctypes.c_int64 * n)(*ao)
    boff = (ctypes.c_int64 * n)(*bo)
    keep = (rk, aoff, boff)
    f = _capi.milo_factors(dtype, n, T, d, ctypes.cast(rk, ctypes.c_void_p), ctypes.cast(aoff, ctypes.c_void_p),
                           ctypes.cast(boff, ctypes.c_void_p), 0x1000, sum(sizes), None, None)
    return f, keep


def test_fetch_validation(L):
    """milo_fetch_blocks checks ids, geometry and offsets on the host."""
    host, keep = _host_set()
    dev, _ = _host_set()
    dev.arena = 0x2000
    ids = lambda *v: ((ctypes.c_int32 * len(v))(*v), len(v))

    def call(h, dv, v):
        arr, n = v
        return L.milo_fetch_blocks(ctypes.byref(h), ctypes.byref(dv), ctypes.cast(arr, ctypes.c_void_p), n, None)

    assert L.milo_fetch_blocks(ctypes.byref(host), ctypes.byref(dev), None, 0, None) == 0  # nothing to do
    assert call(host, dev, ids(4)) == 1 and b"out of range" in L.milo_last_error()
    assert call(host, dev, ids(-1)) == 1
    dev.block_len = 512
    assert call(host, dev, ids(0)) == 1 and b"geometr" in L.milo_last_error()
    dev.block_len = 256
    dev.arena_bytes = host.arena_bytes - 1
    assert call(host, dev, ids(0)) == 1 and b"smaller" in L.milo_last_error()
    dev.arena_bytes = host.arena_bytes
    host.arena_bytes -= 1  # block 3 now reaches past the arena
    dev.arena_bytes = host.arena_bytes
    assert call(host, dev, ids(3)) == 1 and b"past the arena" in L.milo_last_error()
    dev.dtype = 2
    assert call(host, dev, ids(0)) == 1 and b"dtype" in L.milo_last_error()
