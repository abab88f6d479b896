"""fp64 CPU oracle for the MILO hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it, and
it shares no code with the HIP path: the arithmetic lives in ``milo_oracle.c``
(plain C, fp64), this module only marshals numpy arrays in and out and loops
over pools, blocks and sequences.

Method sources, cited by page and section (see the header of ``milo_oracle.c``):
  [REV] evolve.pub review of arXiv 2609.29913 -- Summary, Strengths (Eqs 5-7), FAQ.
  [ABS] shd-paper.top digest -- English abstract, method section.
  [DIG] ai4snews digest -- arXivInterpretation, Figure 1 caption.

Readings of points the pages leave open are stated where they are used.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "milo_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i8p = ctypes.POINTER(ctypes.c_int8)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(force: bool = True) -> str:
    """Compile milo_oracle.c into liboracle.so (gcc, fp64, OpenMP over blocks)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
               "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = load(_LIB_PATH)
    return _lib


def load(path: str):
    """Load an oracle shared library from ``path`` and declare its signatures."""
    L = ctypes.CDLL(path)
    L.oracle_svd_block.argtypes = [_dp, ctypes.c_int, ctypes.c_int, _dp, _dp, ctypes.c_int]
    L.oracle_svd_block.restype = ctypes.c_int
    L.oracle_svd_blocks.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp,
                                    _ip, ctypes.c_int]
    L.oracle_svd_blocks.restype = ctypes.c_int
    L.oracle_allocate.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_double, _ip, _dp]
    L.oracle_allocate.restype = ctypes.c_int64
    L.oracle_objective.argtypes = [_dp, ctypes.c_int, ctypes.c_int, _ip, ctypes.c_double]
    L.oracle_objective.restype = ctypes.c_double
    L.oracle_allocate_uniform.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, _ip]
    L.oracle_allocate_uniform.restype = ctypes.c_int64
    L.oracle_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    L.oracle_splitmix64.restype = ctypes.c_uint64
    L.oracle_allocate_random.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                         ctypes.c_int, _ip]
    L.oracle_allocate_random.restype = ctypes.c_int64
    L.oracle_project.argtypes = [_dp, ctypes.c_int, ctypes.c_int, _dp, ctypes.c_int, _dp, _dp]
    L.oracle_project.restype = None
    L.oracle_reconstruct.argtypes = [_dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp]
    L.oracle_reconstruct.restype = None
    L.oracle_round_bf16.argtypes = [_dp, _dp, ctypes.c_int64]
    L.oracle_round_bf16.restype = None
    L.oracle_round_f32.argtypes = [_dp, _dp, ctypes.c_int64]
    L.oracle_round_f32.restype = None
    L.oracle_quant_int8_rows.argtypes = [_dp, ctypes.c_int, ctypes.c_int, _dp, _i8p, _dp]
    L.oracle_quant_int8_rows.restype = None
    L.oracle_quant_int4_groups.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _i8p, _dp]
    L.oracle_quant_int4_groups.restype = None
    L.oracle_quant_int2_groups.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _u8p, _dp]
    L.oracle_quant_int2_groups.restype = None
    L.oracle_rope.argtypes = [_dp, ctypes.c_int, ctypes.c_double, ctypes.c_double]
    L.oracle_rope.restype = None
    L.oracle_attention.argtypes = [_dp, ctypes.c_int, ctypes.c_int64, _dp, _dp, _i64p,
                                   ctypes.c_int64, ctypes.c_double, ctypes.c_double, _dp]
    L.oracle_attention.restype = ctypes.c_int
    L.oracle_max_threads.argtypes = []
    L.oracle_max_threads.restype = ctypes.c_int
    L.oracle_set_threads.argtypes = [ctypes.c_int]
    L.oracle_set_threads.restype = ctypes.c_int
    return L


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray, typ=_dp):
    return a.ctypes.data_as(typ)


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def set_threads(n: int) -> int:
    """Threads the block loops use from now on; returns the previous count."""
    return int(lib().oracle_set_threads(int(n)))


# --------------------------------------------------------------------------- #
# Step 1: per-block SVD ([REV] Summary: an SVD of each block's K and of its V). #
# --------------------------------------------------------------------------- #
def svd_blocks(X, max_sweeps: int = 60):
    """One-sided Jacobi SVD of each block.

    X: [n, T, d] (any float dtype; widened to fp64).
    Returns (sigma [n, d] descending, V [n, d, d] with V[:, :, i] = v_i, sweeps [n]).
    A sweep count of -1 means the block did not converge within ``max_sweeps``.
    """
    X = _f64(X)
    n, T, d = X.shape
    sigma = np.zeros((n, d))
    V = np.zeros((n, d, d))
    sweeps = np.zeros(n, dtype=np.int32)
    lib().oracle_svd_blocks(_ptr(X), n, T, d, _ptr(sigma), _ptr(V), _ptr(sweeps, _ip), max_sweeps)
    return sigma, V, sweeps


# --------------------------------------------------------------------------- #
# Step 2: greedy rank allocation under a global budget ([REV] Strengths, Eqs 5-7).
# --------------------------------------------------------------------------- #
def allocate(sigma, R: int, eps2: float, k: int | None = None):
    """Literal greedy on the gains log(1 + sigma^2/eps^2) within one pool.

    sigma: [n, k] descending per row.  Returns (rank [n] int32, objective, handed_out).
    """
    sigma = _f64(sigma)
    n, kk = sigma.shape
    if k is not None:
        assert k == kk
    rank = np.zeros(n, dtype=np.int32)
    obj = ctypes.c_double(0.0)
    given = lib().oracle_allocate(_ptr(sigma), n, kk, int(R), float(eps2), _ptr(rank, _ip),
                                  ctypes.byref(obj))
    return rank, float(obj.value), int(given)


POLICIES = ("entropy", "uniform", "random")


def allocate_policy(sigma, R: int, eps2: float, policy: str = "entropy", seed: int = 0,
                    pool: int = 0):
    """Allocation of one pool under `policy`: "entropy" is the greedy of
    ``allocate``; "uniform" and "random" are the equal-budget comparisons
    (oracle_allocate_uniform / oracle_allocate_random).  Returns (rank, objective)."""
    sigma = _f64(sigma)
    n, k = sigma.shape
    if policy == "entropy":
        r, obj, _ = allocate(sigma, R, eps2)
        return r, obj
    rank = np.zeros(n, dtype=np.int32)
    if policy == "uniform":
        lib().oracle_allocate_uniform(n, k, int(R), _ptr(rank, _ip))
    elif policy == "random":
        got = lib().oracle_allocate_random(n, k, int(R), ctypes.c_uint64(seed & (2**64 - 1)), int(pool),
                                           _ptr(rank, _ip))
        if got < 0:
            raise MemoryError("oracle_allocate_random")
    else:
        raise ValueError(policy)
    return rank, objective(sigma, rank, eps2)


def splitmix64(seed: int, c: int) -> int:
    return int(lib().oracle_splitmix64(ctypes.c_uint64(seed & (2**64 - 1)), ctypes.c_uint64(c)))


def objective(sigma, rank, eps2: float) -> float:
    sigma = _f64(sigma)
    n, k = sigma.shape
    rank = np.ascontiguousarray(np.asarray(rank, dtype=np.int32))
    return float(lib().oracle_objective(_ptr(sigma), n, k, _ptr(rank, _ip), float(eps2)))


# --------------------------------------------------------------------------- #
# Step 3: factors A = X V_r, B = V_r^T and their storage encodings.            #
# --------------------------------------------------------------------------- #
def project(X, V, r: int):
    """A = X V[:, :r] (T x r), B = V[:, :r]^T (r x d), fp64."""
    X = _f64(X)
    V = _f64(V)
    T, d = X.shape
    A = np.zeros((T, max(r, 0)))
    B = np.zeros((max(r, 0), d))
    if r > 0:
        lib().oracle_project(_ptr(X), T, d, _ptr(V), r, _ptr(A), _ptr(B))
    return A, B


def reconstruct(A, B):
    A = _f64(A)
    B = _f64(B)
    T, r = A.shape
    r2, d = B.shape
    assert r == r2
    Xh = np.zeros((T, d))
    if r > 0:
        lib().oracle_reconstruct(_ptr(A), _ptr(B), T, r, d, _ptr(Xh))
    return Xh


def round_bf16(x) -> np.ndarray:
    x = _f64(x)
    out = np.empty_like(x)
    lib().oracle_round_bf16(_ptr(x), _ptr(out), x.size)
    return out


def round_f32(x) -> np.ndarray:
    x = _f64(x)
    out = np.empty_like(x)
    lib().oracle_round_f32(_ptr(x), _ptr(out), x.size)
    return out


def quant_int8_rows(M):
    """Per-row absmax INT8.  Returns (scale [rows], codes int8 [rows, cols], dequant fp64)."""
    M = _f64(M)
    if M.ndim != 2:
        raise ValueError("quant_int8_rows expects a 2-D array")
    rows, cols = M.shape
    scale = np.zeros(rows)
    codes = np.zeros((rows, cols), dtype=np.int8)
    deq = np.zeros((rows, cols))
    if rows and cols:
        lib().oracle_quant_int8_rows(_ptr(M), rows, cols, _ptr(scale), _ptr(codes, _i8p), _ptr(deq))
    return scale, codes, deq


I4_GROUP = 32  # elements per 4-bit scale group (tokens of an A row, dims of a B row)


def quant_int4_groups(M, group: int = I4_GROUP):
    """Symmetric 4-bit codes per run of `group` elements of each row.  Returns
    (scale [rows, cols/group], codes int8 in [-7, 7] [rows, cols], dequant fp64)."""
    M = _f64(M)
    if M.ndim != 2:
        raise ValueError("quant_int4_groups expects a 2-D array")
    rows, cols = M.shape
    if cols % group:
        raise ValueError(f"row length {cols} is not a multiple of the group {group}")
    scale = np.zeros((rows, cols // group))
    codes = np.zeros((rows, cols), dtype=np.int8)
    deq = np.zeros((rows, cols))
    if rows and cols:
        lib().oracle_quant_int4_groups(_ptr(M), rows, cols, group, _ptr(scale), _ptr(codes, _i8p), _ptr(deq))
    return scale, codes, deq


I2_GROUP = 32  # elements per 2-bit scale group


def quant_int2_groups(M, group: int = I2_GROUP):
    """Symmetric 2-bit codes per run of `group` elements of each row: s =
    max|x|/3, code c in 0..3 for the nearest level (2c - 3) s.  Returns (scale
    [rows, cols/group], codes uint8 [rows, cols], dequant fp64)."""
    M = _f64(M)
    if M.ndim != 2:
        raise ValueError("quant_int2_groups expects a 2-D array")
    rows, cols = M.shape
    if cols % group:
        raise ValueError(f"row length {cols} is not a multiple of the group {group}")
    scale = np.zeros((rows, cols // group))
    codes = np.zeros((rows, cols), dtype=np.uint8)
    deq = np.zeros((rows, cols))
    if rows and cols:
        lib().oracle_quant_int2_groups(_ptr(M), rows, cols, group, _ptr(scale), _ptr(codes, _u8p), _ptr(deq))
    return scale, codes, deq


def store(A, B, storage: str):
    """Apply the storage encoding to a factor pair; returns the decoded (A, B) in fp64.

    storage: "f32" | "bf16" | "i8" | "i4" | "i2".  For "i8" every row of A (one
    per token) and every row of B (one per rank) gets its own absmax scale.  For
    "i4" and "i2" the rank rows of A^T (T tokens) and of B (d dims) are cut into
    groups of 32 consecutive elements with a scale each.
    """
    if storage == "f32":
        return round_f32(A), round_f32(B)
    if storage == "bf16":
        return round_bf16(A), round_bf16(B)
    if storage == "i8":
        A = _f64(A)
        B = _f64(B)
        if A.shape[1] == 0:
            return A.copy(), B.copy()
        return quant_int8_rows(A)[2], quant_int8_rows(B)[2]
    if storage == "i4":
        A = _f64(A)
        B = _f64(B)
        if A.shape[1] == 0:
            return A.copy(), B.copy()
        return quant_int4_groups(A.T)[2].T.copy(), quant_int4_groups(B)[2]
    if storage == "i2":
        A = _f64(A)
        B = _f64(B)
        if A.shape[1] == 0:
            return A.copy(), B.copy()
        return quant_int2_groups(A.T)[2].T.copy(), quant_int2_groups(B)[2]
    raise ValueError(f"unknown storage {storage!r}")


# --------------------------------------------------------------------------- #
# Step 4: attention over the reconstructed blocks.                             #
# --------------------------------------------------------------------------- #
def rope(x, pos: float, base: float) -> np.ndarray:
    x = _f64(x).copy()
    lib().oracle_rope(_ptr(x), x.shape[-1], float(pos), float(base))
    return x


def attention(q, q_pos: int, K, V, pos, base: float, scale: float) -> np.ndarray:
    """Exact softmax attention of one pre-RoPE query over pre-RoPE keys K [n, d] and values V."""
    q = _f64(q)
    K = _f64(K)
    V = _f64(V)
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    d = q.shape[0]
    n = K.shape[0]
    assert K.shape == (n, d) and V.shape == (n, d) and pos.shape == (n,)
    out = np.zeros(d)
    rc = lib().oracle_attention(_ptr(q), d, int(q_pos), _ptr(K), _ptr(V), _ptr(pos, _i64p), n,
                                float(base), float(scale), _ptr(out))
    if rc != 0:
        raise MemoryError("oracle_attention failed")
    return out


# --------------------------------------------------------------------------- #
# Whole-path helpers used by the tests and the CPU baseline.                   #
# --------------------------------------------------------------------------- #
@dataclass
class Compressed:
    """The oracle's compressed form of a set of blocks (one entry per block)."""
    sigma: np.ndarray                 # [n, d]
    V: np.ndarray                     # [n, d, d]
    rank: np.ndarray                  # [n]
    objective: list                   # per pool
    A: list = field(default_factory=list)   # stored (decoded) A_b, [T, r_b] fp64
    B: list = field(default_factory=list)   # stored (decoded) B_b, [r_b, d] fp64
    sweeps: np.ndarray | None = None


def compress(X, pool_ptr, budgets, eps2: float, storage: str, max_sweeps: int = 60,
             svd=None, policy: str = "entropy", seed: int = 0) -> Compressed:
    """Steps 1-3 for every block.  pool_ptr is the CSR over blocks: pool p holds
    blocks [pool_ptr[p], pool_ptr[p+1]) and gets budget budgets[p].  ``svd`` may
    pass the result of an earlier ``svd_blocks(X)`` to avoid recomputing it."""
    X = _f64(X)
    n, T, d = X.shape
    sigma, V, sweeps = svd if svd is not None else svd_blocks(X, max_sweeps=max_sweeps)
    k = min(T, d)
    rank = np.zeros(n, dtype=np.int32)
    objs = []
    for p in range(len(pool_ptr) - 1):
        lo, hi = int(pool_ptr[p]), int(pool_ptr[p + 1])
        r, obj = allocate_policy(sigma[lo:hi, :k], int(budgets[p]), eps2, policy, seed, p)
        rank[lo:hi] = r
        objs.append(obj)
    out = Compressed(sigma=sigma, V=V, rank=rank, objective=objs, sweeps=sweeps)
    for b in range(n):
        A, B = project(X[b], V[b], int(rank[b]))
        A, B = store(A, B, storage)
        out.A.append(A)
        out.B.append(B)
    return out


def reconstruct_blocks(comp: Compressed, ids=None):
    ids = range(len(comp.A)) if ids is None else ids
    return np.stack([reconstruct(comp.A[b], comp.B[b]) for b in ids])


def decode(q, q_pos, K_blocks, V_blocks, block_len: int, n_kv_heads: int, blocks_per_seq: int,
           sel=None, tail_k=None, tail_v=None, tail_len=None, tail_pos0=None,
           rope_base: float = 1e6, scale: float | None = None) -> np.ndarray:
    """Decode attention for every (sequence, query head).

    q: [batch, Hq, d] pre-RoPE.  K_blocks / V_blocks: callables (or arrays) giving the
    reconstructed pre-RoPE block for factor block id (s*Hkv + h)*blocks_per_seq + b.
    Token t of block b sits at position b*block_len + t; tail token i of sequence s
    at tail_pos0[s] + i.  Query head h reads KV head h // (Hq // Hkv).
    sel: per-sequence list of attended block indices (None = all blocks).
    """
    q = _f64(q)
    batch, Hq, d = q.shape
    G = Hq // n_kv_heads
    scale = (1.0 / np.sqrt(d)) if scale is None else scale
    get_k = K_blocks if callable(K_blocks) else (lambda i: K_blocks[i])
    get_v = V_blocks if callable(V_blocks) else (lambda i: V_blocks[i])
    out = np.zeros((batch, Hq, d))
    for s in range(batch):
        blocks = list(range(blocks_per_seq)) if sel is None else [int(b) for b in sel[s]]
        for h in range(n_kv_heads):
            ks, vs, ps = [], [], []
            for b in blocks:
                fid = (s * n_kv_heads + h) * blocks_per_seq + b
                ks.append(_f64(get_k(fid)))
                vs.append(_f64(get_v(fid)))
                ps.append(np.arange(block_len, dtype=np.int64) + b * block_len)
            if tail_k is not None and tail_len is not None and int(tail_len[s]) > 0:
                L = int(tail_len[s])
                ks.append(_f64(tail_k[s, h, :L]))
                vs.append(_f64(tail_v[s, h, :L]))
                ps.append(np.arange(L, dtype=np.int64) + int(tail_pos0[s]))
            Kc = np.concatenate(ks) if ks else np.zeros((0, d))
            Vc = np.concatenate(vs) if vs else np.zeros((0, d))
            pc = np.concatenate(ps) if ps else np.zeros(0, dtype=np.int64)
            for g in range(G):
                hq = h * G + g
                out[s, hq] = attention(q[s, hq], int(q_pos[s]), Kc, Vc, pc, rope_base, scale)
    return out
