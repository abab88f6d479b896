"""Thin torch-facing binding of libmilo (same names as the C ABI).

PyTorch only supplies device memory and the stream; every step of the path runs
in the HIP library.  Each function marshals tensors into the C structs, calls
the C entry point and raises MiloError on a non-OK status.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _capi as C

_TORCH_TO_MILO = {torch.float32: C.MILO_F32, torch.bfloat16: C.MILO_BF16, torch.int8: C.MILO_I8}
_NAME_TO_MILO = {"f32": C.MILO_F32, "bf16": C.MILO_BF16, "i8": C.MILO_I8, "i4": C.MILO_I4, "i2": C.MILO_I2}
_MILO_TO_TORCH = {C.MILO_F32: torch.float32, C.MILO_BF16: torch.bfloat16, C.MILO_I8: torch.int8}


class MiloError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(message)


class NotConvergedError(MiloError):
    """Raised by milo_compress_blocks(check_convergence=True) when the eigensolve
    of some block reached its iteration cap (a negative entry of sweeps_out)."""

    def __init__(self, blocks):
        self.blocks = list(blocks)
        super().__init__(C.MILO_OK, f"eigensolve reached its iteration cap on {len(self.blocks)} block(s): "
                                    f"{self.blocks[:8]}")


def lib():
    return C.load()


def _check(status: int):
    if status != C.MILO_OK:
        L = lib()
        raise MiloError(status, f"{L.milo_status_string(status).decode()}: "
                                f"{L.milo_last_error().decode()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name: str, dtype=None, numel: int | None = None, optional: bool = False,
          contiguous: bool = True):
    """Marshalling check of a device tensor handed to the library as a plain
    pointer: on a GPU, contiguous, of the element type the C ABI reads, and
    holding at least the elements the call will read or write."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {numel}")


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _torch_stream(stream, device) -> torch.cuda.Stream:
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _on_stream(stream, device, shape, dtype=torch.uint8) -> torch.Tensor:
    """A scratch tensor for work enqueued on `stream`.  It is allocated with that
    stream current, so torch's caching allocator hands its memory, once the
    tensor is dropped, only to later work of the same stream (ordered after the
    kernels that use it), never to another stream's."""
    with torch.cuda.stream(_torch_stream(stream, device)):
        return torch.empty(shape, dtype=dtype, device=device)


def _dtype_code(dtype) -> int:
    if isinstance(dtype, str):
        return _NAME_TO_MILO[dtype]
    return _TORCH_TO_MILO[dtype]


def _host_i32(a):
    arr = (ctypes.c_int32 * len(a))(*[int(v) for v in a])
    return arr


def _host_i64(a):
    arr = (ctypes.c_int64 * len(a))(*[int(v) for v in a])
    return arr


@dataclass
class Factors:
    """Device buffers of one factor set (see milo_factors in include/milo.h)."""
    dtype: str
    n_blocks: int
    block_len: int
    head_dim: int
    rank: torch.Tensor
    a_off: torch.Tensor
    b_off: torch.Tensor
    arena: torch.Tensor
    a_scale: torch.Tensor | None = None
    b_scale: torch.Tensor | None = None

    @staticmethod
    def alloc(dtype: str, n_blocks: int, block_len: int, head_dim: int, arena_bytes: int,
              device="cuda") -> "Factors":
        dev = torch.device(device)
        arena = torch.empty(max(int(arena_bytes), 256), dtype=torch.uint8, device=dev)
        f = Factors(dtype, n_blocks, block_len, head_dim,
                    rank=torch.zeros(n_blocks, dtype=torch.int32, device=dev),
                    a_off=torch.zeros(n_blocks, dtype=torch.int64, device=dev),
                    b_off=torch.zeros(n_blocks, dtype=torch.int64, device=dev),
                    arena=arena)
        if dtype == "i8":
            f.a_scale = torch.zeros(n_blocks * block_len, dtype=torch.float32, device=dev)
            f.b_scale = torch.zeros(n_blocks * head_dim, dtype=torch.float32, device=dev)
        return f

    def struct(self) -> C.milo_factors:
        return C.milo_factors(_NAME_TO_MILO[self.dtype], self.n_blocks, self.block_len,
                              self.head_dim, _p(self.rank), _p(self.a_off), _p(self.b_off),
                              _p(self.arena), self.arena.numel(), _p(self.a_scale),
                              _p(self.b_scale))

    def view(self, lo: int, n: int) -> "Factors":
        """Blocks [lo, lo + n) of this set, sharing its arena (offsets are arena-relative)."""
        return Factors(self.dtype, n, self.block_len, self.head_dim, rank=self.rank[lo:lo + n],
                       a_off=self.a_off[lo:lo + n], b_off=self.b_off[lo:lo + n], arena=self.arena,
                       a_scale=None if self.a_scale is None else
                       self.a_scale[lo * self.block_len:(lo + n) * self.block_len],
                       b_scale=None if self.b_scale is None else
                       self.b_scale[lo * self.head_dim:(lo + n) * self.head_dim])

    def to_host(self) -> "Factors":
        """A copy of this set in pinned host memory (arena, scales and metadata):
        the offloaded form milo_fetch_blocks reads from."""
        def pin(t):
            if t is None:
                return None
            h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
            h.copy_(t)
            return h
        return Factors(self.dtype, self.n_blocks, self.block_len, self.head_dim, rank=pin(self.rank),
                       a_off=pin(self.a_off), b_off=pin(self.b_off), arena=pin(self.arena),
                       a_scale=pin(self.a_scale), b_scale=pin(self.b_scale))

    def like(self, device="cuda") -> "Factors":
        """A set on `device` with this set's layout (metadata copied) and an empty
        arena and scales: the destination of milo_fetch_blocks."""
        dev = torch.device(device)
        f = Factors.alloc(self.dtype, self.n_blocks, self.block_len, self.head_dim, self.arena.numel(),
                          device=dev)
        f.rank.copy_(self.rank)
        f.a_off.copy_(self.a_off)
        f.b_off.copy_(self.b_off)
        return f

    def nbytes(self) -> int:
        """Bytes the factors occupy (arena payload + INT8 scales actually used)."""
        rs = int(self.rank.sum().item())
        if self.dtype == "i4":  # half a byte per element + an fp32 scale per 32 elements
            return rs * (self.block_len + self.head_dim) * 5 // 8
        if self.dtype == "i2":  # a quarter byte per element + an fp32 scale per 32 elements
            return rs * (self.block_len + self.head_dim) * 3 // 8
        used = rs * (self.block_len + self.head_dim) * {"f32": 4, "bf16": 2, "i8": 1}[self.dtype]
        if self.dtype == "i8":
            used += 4 * (self.n_blocks * self.block_len + int(self.rank.sum().item()))
        return used


def milo_profile_enable(on: bool) -> bool:
    return bool(lib().milo_profile_enable(1 if on else 0))


def milo_profile_read() -> dict:
    """{kernel name: (launches, total milliseconds)} since the last read (waits)."""
    cap = 32
    names = (ctypes.c_char_p * cap)()
    cnt = (ctypes.c_int32 * cap)()
    ms = (ctypes.c_double * cap)()
    n = lib().milo_profile_read(names, cnt, ms, cap)
    if n < 0:
        _check(C.MILO_E_HIP)
    return {names[i].decode(): (int(cnt[i]), float(ms[i])) for i in range(min(n, cap))}


def milo_abi_version() -> int:
    return int(lib().milo_abi_version())


def milo_arena_bytes(dtype: str, block_len: int, head_dim: int, pool_ptr, budget) -> int:
    n_pools = len(pool_ptr) - 1
    n = lib().milo_arena_bytes(_NAME_TO_MILO[dtype], block_len, head_dim,
                               ctypes.cast(_host_i32(pool_ptr), ctypes.c_void_p), n_pools,
                               ctypes.cast(_host_i64(budget), ctypes.c_void_p))
    if n == 0 and lib().milo_last_error():
        raise MiloError(C.MILO_E_INVALID, lib().milo_last_error().decode())
    return int(n)


def milo_compress_workspace_bytes(n_blocks: int, block_len: int, head_dim: int = 128) -> int:
    return int(lib().milo_compress_workspace_bytes(n_blocks, block_len, head_dim))


_POLICY = {None: None, "entropy": 0, "uniform": 1, "random": 2}


def _alloc_options(policy, seed):
    code = _POLICY[policy]
    return None if code is None else ctypes.byref(C.milo_alloc_options(code, int(seed) & (2**64 - 1)))


def milo_compress_blocks(x: torch.Tensor, pool_ptr, budget, eps2: float, sigma_out: torch.Tensor,
                         factors: Factors, objective_out: torch.Tensor | None = None,
                         sweeps_out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, row0: torch.Tensor | None = None,
                         row_stride: int | None = None, n_blocks: int | None = None,
                         block_len: int | None = None, stream=None,
                         check_convergence: bool = False) -> None:
    """Compress blocks of ``x``: a contiguous [n_blocks, T, d] tensor, or any tensor
    addressed through ``row0``/``row_stride`` (with n_blocks and block_len given).

    The call is asynchronous, so a block whose eigensolve reached its iteration
    cap shows only as a negative entry of ``sweeps_out`` (which counts the plane
    rotations each block's eigensolve applied).  With
    ``check_convergence=True`` the binding supplies ``sweeps_out`` if none is
    given, waits for the stream and raises NotConvergedError naming such blocks."""
    milo_compress_blocks_ex(x, pool_ptr, budget, eps2, sigma_out, factors, objective_out, sweeps_out,
                            None, 0, workspace, row0, row_stride, n_blocks, block_len, stream,
                            check_convergence)


def milo_compress_blocks_ex(x: torch.Tensor, pool_ptr, budget, eps2: float, sigma_out: torch.Tensor,
                            factors: Factors, objective_out: torch.Tensor | None = None,
                            sweeps_out: torch.Tensor | None = None, policy: str | None = None,
                            seed: int = 0, workspace: torch.Tensor | None = None,
                            row0: torch.Tensor | None = None, row_stride: int | None = None,
                            n_blocks: int | None = None, block_len: int | None = None,
                            stream=None, check_convergence: bool = False) -> None:
    """milo_compress_blocks with the rank allocation policy "entropy" (the
    default), "uniform" or "random" (seeded)."""
    if row0 is None and row_stride is None:
        n_blocks, block_len, d = x.shape
        row_stride = d
    d = factors.head_dim
    if check_convergence and sweeps_out is None:
        sweeps_out = _on_stream(stream, x.device, int(n_blocks), torch.int32)
    _need(x, "x", contiguous=row0 is None)  # with row0 the rows are addressed explicitly
    _need(row0, "row0", torch.int64, int(n_blocks), optional=True)
    _need(sigma_out, "sigma_out", torch.float32, int(n_blocks) * d)
    _need(objective_out, "objective_out", torch.float64, len(pool_ptr) - 1, optional=True)
    _need(sweeps_out, "sweeps_out", torch.int32, int(n_blocks), optional=True)
    _need(workspace, "workspace", torch.uint8, optional=True)
    blocks = C.milo_blocks(_p(x), _dtype_code(x.dtype), _p(row0), int(row_stride), int(n_blocks),
                           int(block_len), int(d))
    fs = factors.struct()
    pp = _host_i32(pool_ptr)
    bb = _host_i64(budget)
    wsb = ctypes.c_size_t(0 if workspace is None else workspace.numel())
    st = lib().milo_compress_blocks_ex(ctypes.byref(blocks), ctypes.cast(pp, ctypes.c_void_p),
                                       len(pool_ptr) - 1, ctypes.cast(bb, ctypes.c_void_p),
                                       float(eps2), _p(sigma_out), _p(objective_out),
                                       ctypes.byref(fs), _p(sweeps_out), _alloc_options(policy, seed),
                                       _p(workspace), ctypes.byref(wsb), _stream(stream))
    if st == C.MILO_E_WORKSPACE and workspace is None:
        workspace = _on_stream(stream, x.device, int(wsb.value))
        return milo_compress_blocks_ex(x, pool_ptr, budget, eps2, sigma_out, factors, objective_out,
                                       sweeps_out, policy, seed, workspace, row0, row_stride,
                                       n_blocks, block_len, stream, check_convergence)
    _check(st)
    if check_convergence and int(n_blocks) > 0:
        _torch_stream(stream, x.device).synchronize()
        bad = torch.nonzero(sweeps_out[:int(n_blocks)] < 0).flatten().tolist()
        if bad:
            raise NotConvergedError(bad)


def milo_allocate_ranks(sigma: torch.Tensor, max_rank: int, pool_ptr, budget, eps2: float,
                        rank_out: torch.Tensor, objective_out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None) -> None:
    milo_allocate_ranks_ex(sigma, max_rank, pool_ptr, budget, eps2, rank_out, objective_out, None, 0,
                           workspace, stream)


def milo_allocate_ranks_ex(sigma: torch.Tensor, max_rank: int, pool_ptr, budget, eps2: float,
                           rank_out: torch.Tensor, objective_out: torch.Tensor | None = None,
                           policy: str | None = None, seed: int = 0,
                           workspace: torch.Tensor | None = None, stream=None) -> None:
    """milo_allocate_ranks with the policy "entropy" (default), "uniform" or "random"."""
    n_blocks, d = sigma.shape
    _need(sigma, "sigma", torch.float32)
    _need(rank_out, "rank_out", torch.int32, n_blocks)
    _need(objective_out, "objective_out", torch.float64, len(pool_ptr) - 1, optional=True)
    _need(workspace, "workspace", torch.uint8, optional=True)
    pp = _host_i32(pool_ptr)
    bb = _host_i64(budget)
    wsb = ctypes.c_size_t(0 if workspace is None else workspace.numel())
    st = lib().milo_allocate_ranks_ex(_p(sigma), n_blocks, d, int(max_rank),
                                      ctypes.cast(pp, ctypes.c_void_p), len(pool_ptr) - 1,
                                      ctypes.cast(bb, ctypes.c_void_p), float(eps2), _p(rank_out),
                                      _p(objective_out), _alloc_options(policy, seed), _p(workspace),
                                      ctypes.byref(wsb), _stream(stream))
    if st == C.MILO_E_WORKSPACE and workspace is None:
        workspace = _on_stream(stream, sigma.device, int(wsb.value))
        return milo_allocate_ranks_ex(sigma, max_rank, pool_ptr, budget, eps2, rank_out,
                                      objective_out, policy, seed, workspace, stream)
    _check(st)


def milo_reconstruct(factors: Factors, block_ids: torch.Tensor, out: torch.Tensor,
                     stream=None, out_off: torch.Tensor | None = None) -> None:
    """Rebuild the listed blocks into out: block i at element offset out_off[i]
    (device int64) when given (milo_reconstruct_ex), else back to back."""
    _need(block_ids, "block_ids", torch.int32)
    n = block_ids.numel()
    rows = factors.block_len * factors.head_dim
    if out_off is None:
        _need(out, "out", None, n * rows)
    else:
        _need(out_off, "out_off", torch.int64, n)
        _need(out, "out", None)
    fs = factors.struct()
    st = lib().milo_reconstruct_ex(ctypes.byref(fs), _p(block_ids), int(n), _p(out), _p(out_off),
                                   _dtype_code(out.dtype), _stream(stream))
    _check(st)


def milo_fetch_blocks(host: Factors, dev: Factors, blocks, stream=None) -> None:
    """Copy the listed blocks' factors from the host-resident set `host` into the
    device set `dev` (same layout); asynchronous on `stream`."""
    for t, name in ((host.rank, "host.rank"), (host.a_off, "host.a_off"), (host.b_off, "host.b_off"),
                    (host.arena, "host.arena")):
        if t.device.type != "cpu":
            raise ValueError(f"{name} must be in host memory")
    if dev.arena.device.type != "cuda":
        raise ValueError("dev.arena must be device memory")
    ids = torch.as_tensor(blocks, dtype=torch.int32).contiguous()
    if ids.device.type != "cpu":
        raise ValueError("blocks must be a host array")
    hs, ds = host.struct(), dev.struct()
    st = lib().milo_fetch_blocks(ctypes.byref(hs), ctypes.byref(ds), _p(ids), int(ids.numel()), _stream(stream))
    _check(st)


def milo_decode_attention(q: torch.Tensor, q_pos: torch.Tensor, k: Factors, v: Factors,
                          blocks_per_seq: int, n_kv_heads: int, out: torch.Tensor,
                          sel_ptr: torch.Tensor | None = None, sel_blk: torch.Tensor | None = None,
                          sel_max: int = 0, tail_k: torch.Tensor | None = None,
                          tail_v: torch.Tensor | None = None, tail_len: torch.Tensor | None = None,
                          tail_pos0: torch.Tensor | None = None, rope_base: float = 1e6,
                          softmax_scale: float | None = None, split_len: int = 0,
                          workspace: torch.Tensor | None = None, stream=None,
                          tail_seg_pos: torch.Tensor | None = None, tail_seg_valid: torch.Tensor | None = None,
                          tail_seg_len: int = 0) -> None:
    batch, n_q, d = q.shape
    _need(q, "q")
    _need(q_pos, "q_pos", torch.int64, batch)
    _need(out, "out", None, batch * n_q * d)
    _need(sel_ptr, "sel_ptr", torch.int32, batch + 1, optional=True)
    _need(sel_blk, "sel_blk", torch.int32, optional=True)
    _need(tail_k, "tail_k", None, optional=True)
    _need(tail_v, "tail_v", None, optional=True)
    segs = tail_seg_pos is not None
    _need(tail_len, "tail_len", torch.int32, batch, optional=tail_k is None or segs)
    _need(tail_pos0, "tail_pos0", torch.int64, batch, optional=tail_k is None or segs)
    _need(workspace, "workspace", torch.uint8, optional=True)
    ks, vs = k.struct(), v.struct()
    tail_cap = 0 if tail_k is None else int(tail_k.shape[2])
    if segs:
        nseg = tail_cap // max(int(tail_seg_len), 1)
        _need(tail_seg_pos, "tail_seg_pos", torch.int64, batch * nseg)
        _need(tail_seg_valid, "tail_seg_valid", torch.int32, batch * nseg)
    args = C.milo_decode_args(
        _p(q), _dtype_code(q.dtype), _p(q_pos), batch, n_q, int(n_kv_heads), d,
        ctypes.pointer(ks), ctypes.pointer(vs), int(blocks_per_seq), _p(sel_ptr), _p(sel_blk),
        int(sel_max), _p(tail_k), _p(tail_v),
        _dtype_code(tail_k.dtype) if tail_k is not None else C.MILO_BF16, tail_cap,
        _p(tail_len), _p(tail_pos0), float(rope_base),
        float(softmax_scale if softmax_scale is not None else d ** -0.5), _p(out),
        _dtype_code(out.dtype), int(split_len), _p(workspace),
        0 if workspace is None else workspace.numel(), _p(tail_seg_pos), _p(tail_seg_valid),
        int(tail_seg_len) if segs else 0)
    need = ctypes.c_size_t(0)
    st = lib().milo_decode_attention(ctypes.byref(args), ctypes.byref(need), _stream(stream))
    if st == C.MILO_E_WORKSPACE and workspace is None:
        workspace = _on_stream(stream, q.device, int(need.value))
        return milo_decode_attention(q, q_pos, k, v, blocks_per_seq, n_kv_heads, out, sel_ptr,
                                     sel_blk, sel_max, tail_k, tail_v, tail_len, tail_pos0,
                                     rope_base, softmax_scale, split_len, workspace, stream,
                                     tail_seg_pos, tail_seg_valid, tail_seg_len)
    _check(st)


def milo_decode_attention_noalloc(q: torch.Tensor, q_pos: torch.Tensor, k: Factors, v: Factors,
                                  blocks_per_seq: int, n_kv_heads: int, out: torch.Tensor,
                                  sel_ptr: torch.Tensor | None = None, sel_blk: torch.Tensor | None = None,
                                  sel_max: int = 0, tail_k: torch.Tensor | None = None,
                                  tail_v: torch.Tensor | None = None, tail_len: torch.Tensor | None = None,
                                  tail_pos0: torch.Tensor | None = None, rope_base: float = 1e6,
                                  softmax_scale: float | None = None, split_len: int = 0,
                                  stream=None) -> None:
    """milo_decode_attention with the library's static per-GPU scratch instead of
    a workspace: nothing is allocated (for callers that cannot allocate)."""
    batch, n_q, d = q.shape
    _need(q, "q")
    _need(q_pos, "q_pos", torch.int64, batch)
    _need(out, "out", None, batch * n_q * d)
    _need(sel_ptr, "sel_ptr", torch.int32, batch + 1, optional=True)
    _need(sel_blk, "sel_blk", torch.int32, optional=True)
    _need(tail_k, "tail_k", None, optional=True)
    _need(tail_v, "tail_v", None, optional=True)
    _need(tail_len, "tail_len", torch.int32, batch, optional=tail_k is None)
    _need(tail_pos0, "tail_pos0", torch.int64, batch, optional=tail_k is None)
    ks, vs = k.struct(), v.struct()
    tail_cap = 0 if tail_k is None else int(tail_k.shape[2])
    args = C.milo_decode_args(
        _p(q), _dtype_code(q.dtype), _p(q_pos), batch, n_q, int(n_kv_heads), d,
        ctypes.pointer(ks), ctypes.pointer(vs), int(blocks_per_seq), _p(sel_ptr), _p(sel_blk),
        int(sel_max), _p(tail_k), _p(tail_v),
        _dtype_code(tail_k.dtype) if tail_k is not None else C.MILO_BF16, tail_cap,
        _p(tail_len), _p(tail_pos0), float(rope_base),
        float(softmax_scale if softmax_scale is not None else d ** -0.5), _p(out),
        _dtype_code(out.dtype), int(split_len), None, 0)
    _check(lib().milo_decode_attention_noalloc(ctypes.byref(args), _stream(stream)))


def reconstruct_then_attend(q: torch.Tensor, q_pos: torch.Tensor, k: Factors, v: Factors,
                            blocks_per_seq: int, n_kv_heads: int, out: torch.Tensor,
                            staging_k: torch.Tensor | None = None,
                            staging_v: torch.Tensor | None = None, staging_dtype=torch.bfloat16,
                            rope_base: float = 1e6, softmax_scale: float | None = None,
                            split_len: int = 0, stream=None, sel=None, tail_k: torch.Tensor | None = None,
                            tail_v: torch.Tensor | None = None, tail_len=None, tail_pos0=None,
                            seg_len: int | None = None):
    """The unfused decode: milo_reconstruct rebuilds the attended blocks into
    token-major staging caches, then milo_decode_attention attends over them as
    an uncompressed cache (no factor blocks).  Returns (staging_k, staging_v).

    Without ``sel`` or a tail every block is attended and the staging caches are
    [batch][n_kv_heads][blocks_per_seq * block_len][head_dim] with block b of
    sequence s, KV head h (factor block (s * n_kv_heads + h) * blocks_per_seq + b)
    at positions b * block_len + t.  With ``sel`` (host lists of ascending,
    distinct block indices per sequence) and/or an uncompressed tail (tail_k,
    tail_v [batch][n_kv_heads][tail_cap][head_dim], host lists tail_len and
    tail_pos0), sequence s's staging row holds its selected blocks in order,
    then a copy of its tail, as segments of ``seg_len`` slots (default: the
    largest multiple of 128 dividing both block_len and tail_cap) whose start
    positions are the blocks' own (b * block_len) and the tail's (tail_pos0),
    so that every key keeps its absolute position."""
    batch = q.shape[0]
    T, d = k.block_len, k.head_dim
    dev = q.device
    if sel is None and tail_k is None:
        shape = (batch, n_kv_heads, blocks_per_seq * T, d)
        if staging_k is None:
            staging_k = _on_stream(stream, dev, shape, staging_dtype)
        if staging_v is None:
            staging_v = _on_stream(stream, dev, shape, staging_dtype)
        _need(staging_k, "staging_k", None, batch * n_kv_heads * blocks_per_seq * T * d)
        _need(staging_v, "staging_v", staging_k.dtype, staging_k.numel())
        with torch.cuda.stream(_torch_stream(stream, dev)):  # scratch of this stream (see _on_stream)
            ids = torch.arange(batch * n_kv_heads * blocks_per_seq, dtype=torch.int32, device=dev)
            tl = torch.full((batch,), blocks_per_seq * T, dtype=torch.int32, device=dev)
            tp = torch.zeros((batch,), dtype=torch.int64, device=dev)
        milo_reconstruct(k, ids, staging_k, stream)
        milo_reconstruct(v, ids, staging_v, stream)
        milo_decode_attention(q, q_pos, k, v, 0, n_kv_heads, out, tail_k=staging_k.view(shape),
                              tail_v=staging_v.view(shape), tail_len=tl, tail_pos0=tp,
                              rope_base=rope_base, softmax_scale=softmax_scale, split_len=split_len,
                              stream=stream)
        return staging_k, staging_v

    sel = [list(range(blocks_per_seq))] * batch if sel is None else [[int(b) for b in x] for x in sel]
    nmax = max((len(x) for x in sel), default=0)
    tcap = 0 if tail_k is None else int(tail_k.shape[2])
    if seg_len is None:
        seg_len = 128
        for c in (2048, 1024, 512, 256):
            if T % c == 0 and tcap % c == 0:
                seg_len = c
                break
    cap = nmax * T + tcap
    shape = (batch, n_kv_heads, cap, d)
    if staging_k is None:
        staging_k = _on_stream(stream, dev, shape, staging_dtype)
    if staging_v is None:
        staging_v = _on_stream(stream, dev, shape, staging_dtype)
    _need(staging_k, "staging_k", None, batch * n_kv_heads * cap * d)
    _need(staging_v, "staging_v", staging_k.dtype, staging_k.numel())
    staging_k, staging_v = staging_k.view(shape), staging_v.view(shape)
    # host-side plan: which blocks land where, and the segment table
    ids, offs = [], []
    nseg = cap // seg_len
    seg_pos = [[0] * nseg for _ in range(batch)]
    seg_valid = [[0] * nseg for _ in range(batch)]
    per_blk = T // seg_len
    for s_, blocks in enumerate(sel):
        for h in range(n_kv_heads):
            for j, b in enumerate(blocks):
                ids.append((s_ * n_kv_heads + h) * blocks_per_seq + b)
                offs.append(((s_ * n_kv_heads + h) * cap + j * T) * d)
        for j, b in enumerate(blocks):
            for u in range(per_blk):
                seg_pos[s_][j * per_blk + u] = b * T + u * seg_len
                seg_valid[s_][j * per_blk + u] = seg_len
        if tcap:
            L = int(tail_len[s_])
            for u in range(tcap // seg_len):
                m = nmax * per_blk + u
                seg_pos[s_][m] = int(tail_pos0[s_]) + u * seg_len
                seg_valid[s_][m] = max(0, min(seg_len, L - u * seg_len))
    with torch.cuda.stream(_torch_stream(stream, dev)):  # scratch of this stream (see _on_stream)
        ids_t = torch.tensor(ids, dtype=torch.int32, device=dev)
        offs_t = torch.tensor(offs, dtype=torch.int64, device=dev)
        sp_t = torch.tensor(seg_pos, dtype=torch.int64, device=dev)
        sv_t = torch.tensor(seg_valid, dtype=torch.int32, device=dev)
        if tcap:  # the uncompressed tail joins the staging rows (data movement only)
            staging_k[:, :, nmax * T:].copy_(tail_k)
            staging_v[:, :, nmax * T:].copy_(tail_v)
    if ids:
        milo_reconstruct(k, ids_t, staging_k, stream, out_off=offs_t)
        milo_reconstruct(v, ids_t, staging_v, stream, out_off=offs_t)
    milo_decode_attention(q, q_pos, k, v, 0, n_kv_heads, out, tail_k=staging_k, tail_v=staging_v,
                          rope_base=rope_base, softmax_scale=softmax_scale, split_len=split_len,
                          stream=stream, tail_seg_pos=sp_t, tail_seg_valid=sv_t, tail_seg_len=seg_len)
    return staging_k, staging_v


def decode_workspace_bytes(q: torch.Tensor, k: Factors, v: Factors, blocks_per_seq: int,
                           n_kv_heads: int, out: torch.Tensor, **kw) -> int:
    """Size query for milo_decode_attention (no work is enqueued)."""
    batch, n_q, d = q.shape
    ks, vs = k.struct(), v.struct()
    tail_k = kw.get("tail_k")
    args = C.milo_decode_args(
        _p(q), _dtype_code(q.dtype), _p(kw.get("q_pos", q)), batch, n_q, int(n_kv_heads), d,
        ctypes.pointer(ks), ctypes.pointer(vs), int(blocks_per_seq), _p(kw.get("sel_ptr")),
        _p(kw.get("sel_blk")), int(kw.get("sel_max", 0)), _p(tail_k), _p(kw.get("tail_v")),
        _dtype_code(tail_k.dtype) if tail_k is not None else C.MILO_BF16,
        0 if tail_k is None else int(tail_k.shape[2]), _p(kw.get("tail_len")),
        _p(kw.get("tail_pos0")), float(kw.get("rope_base", 1e6)), float(d ** -0.5), _p(out),
        _dtype_code(out.dtype), int(kw.get("split_len", 0)), None, 0)
    need = ctypes.c_size_t(0)
    st = lib().milo_decode_attention(ctypes.byref(args), ctypes.byref(need), None)
    if st != C.MILO_E_WORKSPACE:
        _check(st)
    return int(need.value)
