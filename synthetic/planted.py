"""Seeded planted-spectrum KV blocks, queries, block selections and tails.

Each block is X = U diag(s) V^T + E with
  * U (T x d) and V (d x d) the orthonormal Q factors of seeded Gaussian matrices
    (thin QR, R's diagonal positive),
  * s_i = exp(-i / tau_b) for i = 0 .. d-1, tau_b drawn uniformly per block,
  * E Gaussian with standard deviation noise_std (1e-3),
then cast to the storage dtype.  Nothing here depends on the HIP library or on
the oracle; both read the exact tensors returned.
"""
from __future__ import annotations

import hashlib

import torch

from .configs import Config


def derive_seed(*keys) -> int:
    """63-bit seed from an arbitrary tuple of keys (stable across runs and hosts)."""
    h = hashlib.sha256(repr(tuple(keys)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f64": torch.float64}


def _thin_q(Gm: torch.Tensor) -> torch.Tensor:
    """Q of the thin QR of tall Gm [n, m, d] (m >= d) with R's diagonal positive,
    computed as G R^{-1} with R^T R = G^T G (Cholesky); fp64 keeps it orthonormal
    to ~1e-15 for the well-conditioned tall Gaussians used here.  R^{-1} is
    formed explicitly (d x d) so the large product is a plain batched matmul."""
    S = Gm.transpose(-1, -2) @ Gm
    L = torch.linalg.cholesky(S)
    eye = torch.eye(L.shape[-1], dtype=L.dtype, device=L.device).expand_as(L)
    Linv = torch.linalg.solve_triangular(L, eye, upper=False)
    return Gm @ Linv.transpose(-1, -2)


def _square_q(Gm: torch.Tensor) -> torch.Tensor:
    """Q of the QR of square Gm [n, d, d] with diag(R) > 0 (unique), by two
    Cholesky-QR passes in fp64 (CholeskyQR2, orthonormal to ~1e-15 for condition
    numbers up to ~1e7); batches with a Cholesky failure use Householder QR."""
    Q = Gm
    eye = torch.eye(Gm.shape[-1], dtype=Gm.dtype, device=Gm.device).expand_as(Gm)
    for _ in range(2):
        L, info = torch.linalg.cholesky_ex(Q.transpose(-1, -2) @ Q)
        if bool((info != 0).any()):
            Qh, R = torch.linalg.qr(Gm)
            sgn = torch.sign(torch.diagonal(R, dim1=-2, dim2=-1))
            sgn[sgn == 0] = 1
            return Qh * sgn.unsqueeze(-2)
        Q = Q @ torch.linalg.solve_triangular(L, eye, upper=False).transpose(-1, -2)
    return Q


def planted_blocks(n_blocks: int, T: int, d: int, tau_range, seed: int, *,
                   noise_std: float = 1e-3, device="cpu", out_dtype="f32",
                   sub_batch: int = 256, return_tau: bool = False):
    """n_blocks planted blocks [n_blocks, T, d] in ``out_dtype`` ("f32"|"bf16"|"f64")."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    lo, hi = float(tau_range[0]), float(tau_range[1])
    tau = lo + (hi - lo) * torch.rand(n_blocks, generator=gen, device=dev, dtype=torch.float64)
    out = torch.empty((n_blocks, T, d), dtype=_DTYPES[out_dtype], device=dev)
    idx = torch.arange(d, device=dev, dtype=torch.float64)
    for b0 in range(0, n_blocks, sub_batch):
        b1 = min(n_blocks, b0 + sub_batch)
        m = b1 - b0
        U = _thin_q(torch.randn((m, T, d), generator=gen, device=dev, dtype=torch.float64))
        V = _square_q(torch.randn((m, d, d), generator=gen, device=dev, dtype=torch.float64))
        s = torch.exp(-idx.unsqueeze(0) / tau[b0:b1].unsqueeze(1))          # [m, d]
        X = (U * s.unsqueeze(1)) @ V.transpose(-1, -2)
        X += noise_std * torch.randn((m, T, d), generator=gen, device=dev, dtype=torch.float64)
        out[b0:b1] = X.to(out.dtype)
        del U, V, X
    if return_tau:
        return out, tau
    return out


def layer_inputs(cfg: Config, layer: int, kind: str, *, device="cpu", base_seed: int = 20261203,
                 out_dtype: str | None = None, sub_batch: int = 256, return_tau: bool = False):
    """All K (kind="k") or V (kind="v") blocks of one layer, block id
    (s * n_kv_heads + h) * blocks_per_seq + b, as [blocks_per_layer, T, d]."""
    tau = cfg.tau_k if kind == "k" else cfg.tau_v
    seed = derive_seed(base_seed, "blocks", cfg.idx, layer, kind)
    return planted_blocks(cfg.blocks_per_layer, cfg.block_len, cfg.head_dim, tau, seed,
                          noise_std=cfg.noise_std, device=device,
                          out_dtype=out_dtype or cfg.storage, sub_batch=sub_batch,
                          return_tau=return_tau)


def tail_inputs(cfg: Config, layer: int, kind: str, *, device="cpu", base_seed: int = 20261203,
                out_dtype: str | None = None):
    """Uncompressed recent tail [batch, n_kv_heads, tail_len, d] (planted like a block)."""
    if cfg.tail_len == 0:
        return None
    tau = cfg.tau_k if kind == "k" else cfg.tau_v
    seed = derive_seed(base_seed, "tail", cfg.idx, layer, kind)
    x = planted_blocks(cfg.batch * cfg.n_kv_heads, cfg.tail_len, cfg.head_dim, tau, seed,
                       noise_std=cfg.noise_std, device=device, out_dtype=out_dtype or cfg.storage)
    return x.view(cfg.batch, cfg.n_kv_heads, cfg.tail_len, cfg.head_dim)


def queries(cfg: Config, layer: int, *, device="cpu", base_seed: int = 20261203,
            out_dtype: str | None = None, scale: float = 1.0):
    """Pre-RoPE decode queries q ~ N(0, 1) (times ``scale``), [batch, n_q_heads, d]."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(derive_seed(base_seed, "q", cfg.idx, layer))
    q = torch.randn((cfg.batch, cfg.n_q_heads, cfg.head_dim), generator=gen, device=dev,
                    dtype=torch.float64) * scale
    return q.to(_DTYPES[out_dtype or cfg.storage])


def selection(cfg: Config, *, base_seed: int = 20261203):
    """Per sequence, ``sel_blocks`` distinct block indices drawn without replacement
    and sorted (None when every block is attended).  Shared by all layers/heads."""
    if not cfg.sel_blocks:
        return None
    gen = torch.Generator()
    gen.manual_seed(derive_seed(base_seed, "sel", cfg.idx))
    out = []
    for _ in range(cfg.batch):
        perm = torch.randperm(cfg.blocks_per_seq, generator=gen)[: cfg.sel_blocks]
        out.append(sorted(int(x) for x in perm))
    return out
