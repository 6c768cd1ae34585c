"""Seeded synthetic inputs for the attention workloads.

This module draws random numbers, rounds them to the storage dtype and lays out
block tables and pools. It computes none of the method's arithmetic: no
scores, no softmax, no weighted sums, no rotary embedding. Both the oracle side and
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
    "draw_block_tables",
    "alibi_slopes",
    "sink_logits",
    "PrefillCase",
    "DecodeCase",
    "MlaCase",
    "tiny_f32",
    "prefill_case",
    "paged_decode_case",
    "chunked_paged_prefill_case",
    "mla_case",
    "MlaProjCase",
    "mla_proj_case",
    "VarlenPrefillCase",
    "varlen_prefill_case",
    "AppendCase",
    "append_case",
    "MlaAppendCase",
    "mla_append_case",
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
        kshp = (B, cap) + self.k_pool.shape[2:]
        vshp = (B, cap) + self.v_pool.shape[2:]
        kc = np.full(kshp, fill, dtype=np.float32)
        vc = np.full(vshp, fill, dtype=np.float32)
        bs = self.block_size
        for b in range(B):
            L = int(self.seq_lens[b])
            nb = (L + bs - 1) // bs
            ids = self.block_table[b, :nb]
            kc[b, :L] = self.k_pool[ids].reshape((nb * bs,) + kshp[2:])[:L]
            vc[b, :L] = self.v_pool[ids].reshape((nb * bs,) + vshp[2:])[:L]
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
                      max_blocks_per_seq=None, scale=None, seq_lens=None,
                      v_head_dim=None) -> DecodeCase:
    """Paged decode: lengths uniform on ``[len_lo, len_hi]`` (both ends included).

    ``v_head_dim`` (default ``head_dim``) is the width of the V rows."""
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
    vp = _normal(rng, (num_blocks, block_size, n_kv_heads, v_head_dim or head_dim), dtype)
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    return DecodeCase(dtype, q, kp, vp, bt, block_size, seq_lens, n_heads, n_kv_heads,
                      head_dim, float(scale))


def alibi_slopes(n_heads: int) -> np.ndarray:
    """The usual ALiBi slopes for ``n_heads`` heads: ``2^(-8 (h + 1) / n_heads)``."""
    return np.exp2(-8.0 * (np.arange(n_heads) + 1) / n_heads).astype(np.float32)


def sink_logits(seed: int, n_heads: int, std: float = 2.0) -> np.ndarray:
    """Per-head sink logits, N(0, std^2) in float32."""
    return (np.random.default_rng(seed).standard_normal(n_heads) * std).astype(np.float32)


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
             qk_rope_head_dim=64, scale=None, seq_lens=None) -> MlaCase:
    """MLA latent decode: a cache of latent rows ``[c | k_rot]``, every entry iid N(0,1).

    The cache stores ``k_rot`` already rotated at each row's position. A
    rotation of a pair of iid N(0,1) values is again a pair of iid N(0,1)
    values (the standard normal in the plane is rotation invariant), so the
    stored rows of a cache filled by rotating iid draws have exactly this
    distribution; the rotation itself is the append's job. ``q_abs`` is iid
    N(0,1). Default scale is ``1/sqrt(192)``, the un-absorbed query width
    (128 + 64).
    """
    rng = np.random.default_rng(seed)
    W = kv_lora_rank + qk_rope_head_dim
    if seq_lens is None:
        seq_lens = np.full(batch, ctx, dtype=np.int32)
    else:
        seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q = _normal(rng, (batch, n_heads, W), dtype)
    lat = _normal(rng, (batch, ctx, W), dtype)
    if scale is None:
        scale = 1.0 / np.sqrt(192.0)
    return MlaCase(dtype, q, lat, seq_lens, n_heads, kv_lora_rank, qk_rope_head_dim, float(scale))


def _history_rows(bt, held, num_blocks, block_size):
    """[num_blocks, block_size] mask of the pool rows that hold a sequence's history."""
    live = np.zeros((num_blocks, block_size), dtype=bool)
    for b in range(len(held)):
        h = int(held[b])
        full, rest = divmod(h, block_size)
        live[bt[b, :full]] = True
        if rest:
            live[bt[b, full], :rest] = True
    return live


@dataclass
class MlaProjCase:
    """The MLA projections' operands: ``q`` ``[B, H, nope + P]`` (nope first),
    ``k_b`` ``[H, R, nope]`` (absorb direction), ``v_b`` ``[H, v_dim, R]``, and an
    ``o_lat`` ``[B, H, R]`` to up-project on its own."""
    dtype: str
    q: np.ndarray
    k_b: np.ndarray
    v_b: np.ndarray
    o_lat: np.ndarray


def mla_proj_case(seed: int = 0, *, dtype="bf16", batch=32, n_heads=128, qk_nope=128,
                  qk_rope=64, kv_lora_rank=512, v_head_dim=128) -> MlaProjCase:
    """Weights N(0, 1/fan_in) (so outputs keep the inputs' scale), q and o_lat N(0,1)."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (batch, n_heads, qk_nope + qk_rope), dtype)
    k_b = _normal(rng, (n_heads, kv_lora_rank, qk_nope), dtype, qk_nope ** -0.5)
    v_b = _normal(rng, (n_heads, v_head_dim, kv_lora_rank), dtype, kv_lora_rank ** -0.5)
    o_lat = _normal(rng, (batch, n_heads, kv_lora_rank), dtype)
    return MlaProjCase(dtype, q, k_b, v_b, o_lat)


@dataclass
class VarlenPrefillCase:
    """A ragged batch of prefill chunks over one shared cache.

    Sequence ``b`` holds ``seq_kv[b]`` tokens; its chunk is the last
    ``q_lens[b]`` of them (already pushed), at positions
    ``seq_kv[b] - q_lens[b] ..``. ``q`` packs the chunks' query rows
    ``[sum(q_lens), H, D]`` in sequence order; ``cu_q`` is
    ``[0, q_lens[0], q_lens[0] + q_lens[1], ...]``. Paged: ``k``/``v`` are pools
    ``[num_blocks, block_size, Hkv, D]``; contiguous (``block_table`` None):
    ``[B, capacity, Hkv, D]``.
    """
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_q: np.ndarray
    seq_kv: np.ndarray
    n_heads: int
    n_kv_heads: int
    head_dim: int
    scale: float
    block_table: Optional[np.ndarray] = None
    block_size: int = 0

    @property
    def batch(self) -> int:
        return len(self.seq_kv)

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_q)


def varlen_prefill_case(seed: int = 0, *, dtype="bf16", q_lens=None, cached=None, batch=16,
                        q_lo=1, q_hi=1024, cached_lo=0, cached_hi=4096, n_heads=32, n_kv_heads=8,
                        head_dim=128, block_size=16, paged=True, scale=None, slack=0.10,
                        std=1.0) -> VarlenPrefillCase:
    """Ragged chunks: ``q_lens`` ~ U[q_lo, q_hi] new tokens after ``cached`` ~ U[cached_lo,
    cached_hi] cached ones per sequence (both ends included), unless given."""
    rng = np.random.default_rng(seed)
    if q_lens is None:
        q_lens = rng.integers(q_lo, q_hi + 1, size=batch)
    if cached is None:
        cached = rng.integers(cached_lo, cached_hi + 1, size=len(q_lens))
    q_lens = np.asarray(q_lens, dtype=np.int64)
    cached = np.asarray(cached, dtype=np.int64)
    seq_kv = (q_lens + cached).astype(np.int32)
    B = len(q_lens)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    row = (n_kv_heads, head_dim)
    if paged:
        nb, bt = draw_block_tables(rng, seq_kv, block_size, slack)
        k = _normal(rng, (nb, block_size) + row, dtype, std)
        v = _normal(rng, (nb, block_size) + row, dtype, std)
    else:
        bt = None
        cap = int(seq_kv.max())
        k = _normal(rng, (B, cap) + row, dtype, std)
        v = _normal(rng, (B, cap) + row, dtype, std)
    q = _normal(rng, (int(cu_q[-1]), n_heads, head_dim), dtype, std)
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    return VarlenPrefillCase(dtype, q, k, v, cu_q, seq_kv, n_heads, n_kv_heads, head_dim,
                             float(scale), bt, block_size if paged else 0)


@dataclass
class AppendCase:
    """One push into a KV cache: ``n_new`` rows per sequence after ``held[b]`` rows.

    ``k_new``/``v_new`` are ``[B, n_new, Hkv, D]``. Paged: the pools
    ``[num_blocks, block_size, Hkv, D]`` with tables that already reserve the
    blocks the new rows need; contiguous: ``[B, capacity, Hkv, D]``. Cache rows
    not yet written hold NaN.
    """
    dtype: str
    k_new: np.ndarray
    v_new: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    held: np.ndarray
    block_table: Optional[np.ndarray]
    block_size: int


def append_case(seed: int = 0, *, dtype="bf16", batch=64, n_new=1, held_lo=511, held_hi=8191,
                n_kv_heads=8, head_dim=128, block_size=16, paged=True, held=None) -> AppendCase:
    """A push of ``n_new`` tokens per sequence; ``held`` ~ U[held_lo, held_hi] rows already cached.

    The default is the paged-decode workload's push: 64 sequences that hold
    511..8191 rows each receive this step's K/V row (so they hold 512..8192
    after the push). History rows are iid N(0,1) in the storage dtype; rows
    past the history are NaN.
    """
    rng = np.random.default_rng(seed)
    if held is None:
        held = rng.integers(held_lo, held_hi + 1, size=batch).astype(np.int32)
    else:
        held = np.asarray(held, dtype=np.int32)
    after = held.astype(np.int64) + n_new
    row = (n_kv_heads, head_dim)
    if paged:
        maxb = int((after.max() + block_size - 1) // block_size)
        nb, bt = draw_block_tables(rng, after, block_size, 0.10, maxb)
        kc = _normal(rng, (nb, block_size) + row, dtype)
        vc = _normal(rng, (nb, block_size) + row, dtype)
        live = _history_rows(bt, held, nb, block_size)
        kc[~live] = np.nan
        vc[~live] = np.nan
    else:
        bt = None
        cap = int(after.max())
        kc = np.full((batch, cap) + row, np.nan, dtype=np.float32)
        vc = np.full((batch, cap) + row, np.nan, dtype=np.float32)
        for b in range(batch):
            kc[b, :held[b]] = _normal(rng, (int(held[b]),) + row, dtype)
            vc[b, :held[b]] = _normal(rng, (int(held[b]),) + row, dtype)
    k_new = _normal(rng, (batch, n_new) + row, dtype)
    v_new = _normal(rng, (batch, n_new) + row, dtype)
    return AppendCase(dtype, k_new, v_new, kc, vc, held, bt, block_size if paged else 0)


@dataclass
class MlaAppendCase:
    """One latent push per sequence: ``c_new`` ``[B, R]`` and ``k_rot_new`` ``[B, P]`` (unrotated)
    into a latent cache (``[B, capacity, R + P]``, or a pool ``[num_blocks, block_size, R + P]``
    with ``block_table``) that holds ``held[b]`` rows; later rows are NaN."""
    dtype: str
    c_new: np.ndarray
    k_rot_new: np.ndarray
    latent: np.ndarray
    held: np.ndarray
    block_table: Optional[np.ndarray]
    block_size: int
    theta: float


def mla_append_case(seed: int = 0, *, dtype="bf16", batch=32, held_lo=4095, held_hi=4095,
                    kv_lora_rank=512, qk_rope_head_dim=64, theta=10000.0, paged=False,
                    block_size=16, capacity=None, held=None) -> MlaAppendCase:
    """The MLA decode workload's push: 32 sequences holding 4095 rows get their 4096th."""
    rng = np.random.default_rng(seed)
    W = kv_lora_rank + qk_rope_head_dim
    if held is None:
        held = rng.integers(held_lo, held_hi + 1, size=batch).astype(np.int32)
    else:
        held = np.asarray(held, dtype=np.int32)
    after = held.astype(np.int64) + 1
    if paged:
        maxb = int((after.max() + block_size - 1) // block_size)
        nb, bt = draw_block_tables(rng, after, block_size, 0.10, maxb)
        lat = _normal(rng, (nb, block_size, W), dtype)
        lat[~_history_rows(bt, held, nb, block_size)] = np.nan
    else:
        bt = None
        cap = int(after.max()) if capacity is None else int(capacity)
        lat = np.full((batch, cap, W), np.nan, dtype=np.float32)
        for b in range(batch):
            lat[b, :held[b]] = _normal(rng, (int(held[b]), W), dtype)
    c_new = _normal(rng, (batch, kv_lora_rank), dtype)
    k_rot_new = _normal(rng, (batch, qk_rope_head_dim), dtype)
    return MlaAppendCase(dtype, c_new, k_rot_new, lat, held, bt, block_size if paged else 0,
                         float(theta))


CONFIG_DESCRIPTIONS = {
    "tiny_f32": "causal GQA fp32, H=4 Hkv=2 D=16, prefill 64 at offset 0 then 8 decode steps, scale 1/4",
    "prefill_bf16": "causal GQA prefill bf16, B=1 H=28 Hkv=4 D=128 seq_q=seq_kv=4096 offset 0, "
                    "N(0,1)/sqrt(2), scale 1/sqrt(128)",
    "paged_decode_bf16": "paged GQA decode bf16, 64 seqs, seq_lens U[512,8192], H=32 Hkv=8 D=128 "
                         "block_size 16, pool = blocks needed + 10%, N(0,1), scale 1/sqrt(128)",
    "chunked_prefill_paged_bf16": "chunked prefill on paged KV bf16, 8 seqs, 3584 cached + 512 new, "
                                  "H=32 Hkv=8 D=128 block_size 16, scale 0.05, N(0,1)",
    "mla_decode_bf16": "MLA absorbed latent decode bf16, 32 seqs x 4096 ctx, H=128, latent 576 = "
                       "512 + 64 (stored rows iid N(0,1)), scale 1/sqrt(192)",
    "varlen_prefill_paged_bf16": "ragged chunked prefill bf16 over one paged pool: 16 seqs, chunk "
                                 "U[1,1024] after U[0,4096] cached, H=32 Hkv=8 D=128 block 16, "
                                 "scale 1/sqrt(128), N(0,1)",
    "mla_proj_bf16": "MLA absorb q_nope.k_b[h] and up-projection v_b[h].o_lat, bf16, 32 seqs, "
                     "H=128, qk_nope 128, rope 64, R 512, v_head_dim 128, weights N(0,1/fan_in)",
    "append_paged_bf16": "push of this step's K/V row into the paged-decode pool: 64 seqs holding "
                         "511..8191 rows, Hkv=8 D=128 block 16",
    "mla_append_bf16": "push of the 4096th latent row [c | rope(k_rot)] for 32 seqs, R=512 P=64, "
                       "theta 1e4",
}
