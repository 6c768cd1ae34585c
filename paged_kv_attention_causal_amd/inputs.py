"""Seeded synthetic inputs for the attention workloads.

This module draws random numbers, rounds them to the storage dtype, lays out
block tables and pools, and rotates the ``k_rot`` slice of an MLA latent row
(the latent cache stores that slice already rotated). It computes no
attention: no scores, no softmax, no weighted sums. Both the oracle side and
the GPU side of every test and benchmark read the arrays it returns, so the
two always see the same stored values.

Every array is returned as ``float32``. For a ``"bf16"`` case the values are
already rounded to bfloat16 (round to nearest, ties to even), so casting them
to a bfloat16 tensor is exact and upcasting them to float64 gives the very
values the GPU reads.

Draw order inside one case is fixed: sequence lengths, then the pool
permutation, then Q, then K, then V (MLA: Q, then the latent). All draws come
from ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "bf16_round",
    "to_storage",
    "rope_interleaved",
    "draw_block_tables",
    "PrefillCase",
    "DecodeCase",
    "MlaCase",
    "tiny_f32",
    "prefill_case",
    "paged_decode_case",
    "chunked_paged_prefill_case",
    "mla_case",
    "CONFIG_DESCRIPTIONS",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), by bits.

    Returns float32 values whose low 16 bits are zero. NaN stays NaN; values
    that round past the largest finite bfloat16 become infinity, as IEEE
    rounding requires.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = (x.view(np.uint32)[nan] | np.uint32(0x00400000)) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round ``x`` to the storage dtype (``"f32"`` or ``"bf16"``), kept as float32."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(x)
    if dtype == "bf16":
        return bf16_round(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def rope_interleaved(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Interleaved rotary embedding on the last axis of ``x``, in float64.

    The last axis holds pairs ``(x[2i], x[2i+1])``; pair ``i`` at position
    ``t`` is rotated by the angle ``t * theta**(-2i/d)``, ``d`` being the
    last-axis width. ``positions`` broadcasts against ``x.shape[:-1]``.
    This is the pair layout that frink-models 0.31.0 ``src/mla/mod.rs``
    calls interleaved (module doc, point 2, and ``rotate_pe``).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("rotary width must be even")
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / d)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def draw_block_tables(rng: np.random.Generator, seq_lens, block_size: int,
                      slack: float = 0.10, max_blocks_per_seq: Optional[int] = None):
    """Random non-overlapping block tables over a shared pool.

    The pool holds ``ceil((1 + slack) * total)`` blocks, ``total`` being the
    blocks the sequences need; a random permutation of the pool is dealt to
    the sequences in order, and the leftover blocks stay unused. Unused table
    entries are ``-1``. Returns ``(num_blocks, block_table[int32])``.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    need = (seq_lens + block_size - 1) // block_size
    total = int(need.sum())
    num_blocks = int(np.ceil((1.0 + slack) * total - 1e-9))
    if max_blocks_per_seq is None:
        max_blocks_per_seq = int(need.max())
    perm = rng.permutation(num_blocks)
    bt = np.full((len(seq_lens), max_blocks_per_seq), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[off:off + n]
        off += n
    return num_blocks, bt


def _normal(rng, shape, dtype, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return to_storage(x, dtype)


@dataclass
class PrefillCase:
    """Multi-token causal prefill over a contiguous or paged K/V.

    ``q`` is ``[B, seq_q, H, D]``. Contiguous: ``k``/``v`` are
    ``[B, kv_capacity, Hkv, D]``. Paged: ``k``/``v`` are pools
    ``[num_blocks, block_size, Hkv, D]`` and ``block_table`` is
    ``[B, max_blocks_per_seq]``.
    """
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    n_heads: int
    n_kv_heads: int
    head_dim: int
    seq_q: int
    seq_kv: int
    position_offset: int
    scale: float
    block_table: Optional[np.ndarray] = None
    block_size: int = 0

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def paged(self) -> bool:
        return self.block_table is not None


@dataclass
class DecodeCase:
    """Single-token decode: ``q`` is ``[B, H, D]``; ``seq_lens[b]`` keys per sequence.

    Paged: ``k_pool``/``v_pool`` are ``[num_blocks, block_size, Hkv, D]``.
    ``contig()`` lays the same rows out as ``[B, capacity, Hkv, D]``.
    """
    dtype: str
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_table: np.ndarray
    block_size: int
    seq_lens: np.ndarray
    n_heads: int
    n_kv_heads: int
    head_dim: int
    scale: float

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    def contig(self, capacity: Optional[int] = None, fill: float = 0.0):
        """The same cache rows as a contiguous ``[B, capacity, Hkv, D]`` cache.

        Rows past a sequence's length hold ``fill`` (pass NaN to poison them).
        """
        cap = int(self.seq_lens.max()) if capacity is None else int(capacity)
        B = self.batch
        shp = (B, cap) + self.k_pool.shape[2:]
        kc = np.full(shp, fill, dtype=np.float32)
        vc = np.full(shp, fill, dtype=np.float32)
        bs = self.block_size
        for b in range(B):
            L = int(self.seq_lens[b])
            nb = (L + bs - 1) // bs
            ids = self.block_table[b, :nb]
            kc[b, :L] = self.k_pool[ids].reshape((nb * bs,) + shp[2:])[:L]
            vc[b, :L] = self.v_pool[ids].reshape((nb * bs,) + shp[2:])[:L]
        return kc, vc


@dataclass
class MlaCase:
    """Absorbed MLA latent decode.

    ``q_abs`` is ``[B, H, R + P]`` (absorbed part, then the rotary part);
    ``latent`` is ``[B, capacity, R + P]`` with rows ``[c (R) | k_rot (P)]``.
    """
    dtype: str
    q_abs: np.ndarray
    latent: np.ndarray
    seq_lens: np.ndarray
    n_heads: int
    kv_lora_rank: int
    qk_rope_head_dim: int
    scale: float

    @property
    def batch(self) -> int:
        return self.q_abs.shape[0]


def tiny_f32(seed: int = 0, n_heads=4, n_kv_heads=2, head_dim=16, prefill_len=64, decode_steps=8):
    """Tiny causal GQA in fp32: one sequence of ``prefill_len + decode_steps`` tokens.

    Returns ``(q, k, v, scale)`` with ``q`` ``[1, T, H, D]`` and ``k``/``v``
    ``[1, T, Hkv, D]``, ``T = prefill_len + decode_steps``. The prefill uses
    the first ``prefill_len`` rows; decode step ``s`` uses query row
    ``prefill_len + s`` over the first ``prefill_len + s + 1`` cache rows.
    """
    rng = np.random.default_rng(seed)
    T = prefill_len + decode_steps
    q = _normal(rng, (1, T, n_heads, head_dim), "f32")
    k = _normal(rng, (1, T, n_kv_heads, head_dim), "f32")
    v = _normal(rng, (1, T, n_kv_heads, head_dim), "f32")
    return q, k, v, 1.0 / np.sqrt(head_dim)


def prefill_case(seed: int = 0, *, dtype="bf16", batch=1, n_heads=28, n_kv_heads=4, head_dim=128,
                 seq_q=4096, position_offset=0, std=2.0 ** -0.5, scale=None,
                 kv_capacity=None) -> PrefillCase:
    """Causal prefill over a contiguous cache: ``seq_kv = position_offset + seq_q``."""
    rng = np.random.default_rng(seed)
    seq_kv = position_offset + seq_q
    cap = seq_kv if kv_capacity is None else kv_capacity
    q = _normal(rng, (batch, seq_q, n_heads, head_dim), dtype, std)
    k = _normal(rng, (batch, cap, n_kv_heads, head_dim), dtype, std)
    v = _normal(rng, (batch, cap, n_kv_heads, head_dim), dtype, std)
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    return PrefillCase(dtype, q, k, v, n_heads, n_kv_heads, head_dim, seq_q, seq_kv,
                       position_offset, float(scale))


def paged_decode_case(seed: int = 0, *, dtype="bf16", batch=64, len_lo=512, len_hi=8192,
                      n_heads=32, n_kv_heads=8, head_dim=128, block_size=16, slack=0.10,
                      max_blocks_per_seq=None, scale=None, seq_lens=None) -> DecodeCase:
    """Paged decode: lengths uniform on ``[len_lo, len_hi]`` (both ends included)."""
    rng = np.random.default_rng(seed)
    if seq_lens is None:
        seq_lens = rng.integers(len_lo, len_hi + 1, size=batch).astype(np.int32)
    else:
        seq_lens = np.asarray(seq_lens, dtype=np.int32)
    if max_blocks_per_seq is None:
        max_blocks_per_seq = (len_hi + block_size - 1) // block_size
    num_blocks, bt = draw_block_tables(rng, seq_lens, block_size, slack, max_blocks_per_seq)
    q = _normal(rng, (batch, n_heads, head_dim), dtype)
    kp = _normal(rng, (num_blocks, block_size, n_kv_heads, head_dim), dtype)
    vp = _normal(rng, (num_blocks, block_size, n_kv_heads, head_dim), dtype)
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    return DecodeCase(dtype, q, kp, vp, bt, block_size, seq_lens, n_heads, n_kv_heads,
                      head_dim, float(scale))


def chunked_paged_prefill_case(seed: int = 0, *, dtype="bf16", batch=8, cached=3584, seq_q=512,
                               n_heads=32, n_kv_heads=8, head_dim=128, block_size=16,
                               slack=0.10, scale=0.05) -> PrefillCase:
    """A new chunk of ``seq_q`` tokens after ``cached`` tokens, K/V in a paged pool.

    The chunk's own K/V rows are already in the pool (they are appended
    before attending), so ``seq_kv = cached + seq_q`` for every sequence.
    """
    rng = np.random.default_rng(seed)
    seq_kv = cached + seq_q
    lens = np.full(batch, seq_kv, dtype=np.int64)
    num_blocks, bt = draw_block_tables(rng, lens, block_size, slack)
    q = _normal(rng, (batch, seq_q, n_heads, head_dim), dtype)
    kp = _normal(rng, (num_blocks, block_size, n_kv_heads, head_dim), dtype)
    vp = _normal(rng, (num_blocks, block_size, n_kv_heads, head_dim), dtype)
    return PrefillCase(dtype, q, kp, vp, n_heads, n_kv_heads, head_dim, seq_q, seq_kv, cached,
                       float(scale), block_table=bt, block_size=block_size)


def mla_case(seed: int = 0, *, dtype="bf16", batch=32, ctx=4096, n_heads=128, kv_lora_rank=512,
             qk_rope_head_dim=64, theta=10000.0, scale=None, seq_lens=None) -> MlaCase:
    """MLA latent decode: latent rows ``[c | k_rot]`` with ``k_rot`` rotated at its position.

    ``c`` and the pre-rotation ``k_rot`` are iid N(0,1); the rotation runs in
    float64 at each row's own position, then the row is rounded to the
    storage dtype. ``q_abs`` is iid N(0,1). Default scale is ``1/sqrt(192)``,
    the un-absorbed query width (128 + 64).
    """
    rng = np.random.default_rng(seed)
    W = kv_lora_rank + qk_rope_head_dim
    if seq_lens is None:
        seq_lens = np.full(batch, ctx, dtype=np.int32)
    else:
        seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q = _normal(rng, (batch, n_heads, W), dtype)
    lat = rng.standard_normal(size=(batch, ctx, W), dtype=np.float32)
    pos = np.arange(ctx, dtype=np.float64)[None, :]
    lat[..., kv_lora_rank:] = rope_interleaved(lat[..., kv_lora_rank:], pos, theta).astype(np.float32)
    lat = to_storage(lat, dtype)
    if scale is None:
        scale = 1.0 / np.sqrt(192.0)
    return MlaCase(dtype, q, lat, seq_lens, n_heads, kv_lora_rank, qk_rope_head_dim, float(scale))


CONFIG_DESCRIPTIONS = {
    "tiny_f32": "causal GQA fp32, H=4 Hkv=2 D=16, prefill 64 at offset 0 then 8 decode steps, scale 1/4",
    "prefill_bf16": "causal GQA prefill bf16, B=1 H=28 Hkv=4 D=128 seq_q=seq_kv=4096 offset 0, "
                    "N(0,1)/sqrt(2), scale 1/sqrt(128)",
    "paged_decode_bf16": "paged GQA decode bf16, 64 seqs, seq_lens U[512,8192], H=32 Hkv=8 D=128 "
                         "block_size 16, pool = blocks needed + 10%, N(0,1), scale 1/sqrt(128)",
    "chunked_prefill_paged_bf16": "chunked prefill on paged KV bf16, 8 seqs, 3584 cached + 512 new, "
                                  "H=32 Hkv=8 D=128 block_size 16, scale 0.05, N(0,1)",
    "mla_decode_bf16": "MLA absorbed latent decode bf16, 32 seqs x 4096 ctx, H=128, latent 576 = "
                       "512 + 64 rotated (theta 1e4), scale 1/sqrt(192), N(0,1)",
}
