"""Plain float64 CPU oracle for causal grouped-query attention over a KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it. It shares no code with the HIP
library and imports nothing from it.

What it computes is the plain definition of causal GQA, written out step by
step in the order kopitiam-runtime 0.2.4 ``src/attention.rs`` gives it in
``attention_forward`` (its attention core, after the projections and RoPE):
repeat each KV head ``group_size`` times, take ``scale * Q K^T``, add the
additive 0/-inf causal mask, take a row softmax, multiply by V. The KV heads
are repeated by materialising a copy, the mask is a real array of 0 and
-inf, and the softmax is the textbook ``exp(s - max) / sum``: no blocking, no
online rescaling, no fusion.

Inputs are NumPy arrays holding the exact values the GPU reads (fp32, or fp32
holding bf16-rounded values); everything is upcast to float64 here, so input
quantisation never counts as error.

Readings of the pages used here (each also listed in the design doc):
* ``scale`` is the whole logit multiplier. kopitiam divides by sqrt(head_dim);
  frink-models 0.31.0 ``src/mla/mod.rs`` (``absorbed_attention``) passes an
  explicit scale; this oracle takes it as an argument and ``1/sqrt(D)``
  reproduces kopitiam.
* Decode is push-then-attend: the query at position ``L-1`` sees its own key
  (frink-models 0.38.0 ``src/decoder/attn_block.rs``,
  ``push_and_attend_row``; kopitiam's module doc, "Causal masking").
* A paged cache holds token ``t`` of sequence ``b`` at
  ``pool[block_table[b][t // block_size]][t % block_size]`` (the pages show
  only ``block_table()`` and ``seq_len()``; this is the plain reading).
* MLA: the key of every head is the whole latent row ``[c | k_rot]`` and the
  value is its first ``kv_lora_rank`` entries (``absorbed_attention`` in
  frink-models 0.31.0 ``src/mla/mod.rs``).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "repeat_kv_heads",
    "causal_mask",
    "masked_softmax",
    "gqa_attention",
    "gather_paged",
    "prefill",
    "decode_contig",
    "decode_paged",
    "mla_decode_latent",
    "mla_naive",
    "mla_absorb_q",
    "mla_up_proj",
    "mla_absorbed",
    "prefill_varlen",
    "gqa_attention_arms",
    "decode_arms",
    "rope_interleaved",
    "append_rows",
    "mla_append_latent",
]


def repeat_kv_heads(x: np.ndarray, group_size: int) -> np.ndarray:
    """``[n_kv, seq, D]`` -> ``[n_kv * group_size, seq, D]``, each KV head repeated contiguously.

    Query head ``g`` reads KV head ``g // group_size``; ``group_size == 1``
    returns the input unchanged (kopitiam-runtime 0.2.4 ``src/attention.rs``,
    ``repeat_kv_heads``).
    """
    x = np.asarray(x)
    if group_size == 1:
        return x
    n_kv, seq, d = x.shape
    out = np.broadcast_to(x[:, None, :, :], (n_kv, group_size, seq, d))
    return np.ascontiguousarray(out).reshape(n_kv * group_size, seq, d)


def causal_mask(seq_q: int, seq_kv: int, position_offset: int) -> np.ndarray:
    """Additive bias ``[1, seq_q, seq_kv]``: 0 where key ``j <= position_offset + i``, -inf elsewhere.

    Query row ``i`` sits at absolute position ``position_offset + i``; key
    column ``j`` is absolute position ``j`` (kopitiam-runtime 0.2.4
    ``src/attention.rs``, ``causal_mask``).
    """
    m = np.zeros((1, seq_q, seq_kv), dtype=np.float64)
    for i in range(seq_q):
        last_visible = position_offset + i
        m[0, i, last_visible + 1:] = -np.inf
    return m


def masked_softmax(scores: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Softmax over the last axis of ``scores + mask``: ``exp(s - max) / sum``.

    A masked entry is exactly -inf, so its weight is exactly 0.
    """
    s = np.asarray(scores, dtype=np.float64) + mask
    mx = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - mx)
    return e / np.sum(e, axis=-1, keepdims=True)


def gqa_attention(q, k, v, n_heads: int, n_kv_heads: int, position_offset: int,
                  scale: float) -> np.ndarray:
    """Causal GQA for one sequence, in float64.

    ``q`` is ``[seq_q, H, D]``, ``k``/``v`` are ``[seq_kv, Hkv, Dv]``
    (``Dv`` may differ from ``D`` for ``v``). Returns ``[seq_q, H, Dv]``.
    The steps follow kopitiam's ``attention_forward``: to head-major,
    repeat KV heads, ``scale * Q K^T``, add the causal mask, row softmax,
    ``P V``, back to token-major.
    """
    if n_kv_heads <= 0 or n_heads <= 0 or n_heads % n_kv_heads != 0:
        raise ValueError("n_heads must be a positive multiple of n_kv_heads")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    seq_q, seq_kv = q.shape[0], k.shape[0]
    group_size = n_heads // n_kv_heads
    qh = q.transpose(1, 0, 2)                   # [H, seq_q, D]
    kh = k.transpose(1, 0, 2)                   # [Hkv, seq_kv, D]
    vh = v.transpose(1, 0, 2)                   # [Hkv, seq_kv, Dv]
    k_rep = repeat_kv_heads(kh, group_size)     # [H, seq_kv, D]
    v_rep = repeat_kv_heads(vh, group_size)     # [H, seq_kv, Dv]
    scores = np.matmul(qh, k_rep.transpose(0, 2, 1)) * scale   # [H, seq_q, seq_kv]
    probs = masked_softmax(scores, causal_mask(seq_q, seq_kv, position_offset))
    out = np.matmul(probs, v_rep)               # [H, seq_q, Dv]
    return out.transpose(1, 0, 2)


def gqa_attention_arms(q, k, v, n_heads: int, n_kv_heads: int, position_offset: int,
                       scale: float, window: int = 0, softcap: float = 0.0, alibi=None,
                       sinks=None) -> np.ndarray:
    """Causal GQA with the optional arms of one attention layer, in float64.

    The arms frink-models 0.38.0 ``src/decoder/attn_block.rs``
    (``push_and_attend_row``) hands its one kernel besides the plain case,
    read as their usual definitions (the page names them, it does not spell
    them out):
    * ``window > 0``: row ``i`` (position ``p = position_offset + i``) sees
      only keys ``j`` with ``p - window < j <= p``;
    * ``softcap > 0``: every logit ``x = scale * q.k`` becomes
      ``softcap * tanh(x / softcap)``;
    * ``alibi`` (``[H]`` slopes): head ``h`` adds ``alibi[h] * (j - p)`` to
      its logits after the softcap;
    * ``sinks`` (``[H]`` logits): head ``h``'s softmax runs over its visible
      keys plus one extra logit ``sinks[h]`` that carries no value, so the
      weights of the keys sum to less than one.
    ``k`` is ``[seq_kv, Hkv, D]``, ``v`` is ``[seq_kv, Hkv, Dv]`` (``Dv`` may
    differ from ``D``: the page's ``head_dim`` and ``v_head_dim``). Returns
    ``[seq_q, H, Dv]``. The steps: head-major, repeat the KV heads, scores,
    softcap, ALiBi bias, additive mask (causal and window), softmax with the
    sink, ``P V``.
    """
    if n_kv_heads <= 0 or n_heads <= 0 or n_heads % n_kv_heads != 0:
        raise ValueError("n_heads must be a positive multiple of n_kv_heads")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    seq_q, seq_kv = q.shape[0], k.shape[0]
    group_size = n_heads // n_kv_heads
    qh = q.transpose(1, 0, 2)
    k_rep = repeat_kv_heads(k.transpose(1, 0, 2), group_size)
    v_rep = repeat_kv_heads(v.transpose(1, 0, 2), group_size)
    x = np.matmul(qh, k_rep.transpose(0, 2, 1)) * scale          # [H, seq_q, seq_kv]
    if softcap > 0:
        x = softcap * np.tanh(x / softcap)
    pos = position_offset + np.arange(seq_q)[:, None]            # [seq_q, 1]
    rel = np.arange(seq_kv)[None, :] - pos                       # j - p
    if alibi is not None:
        x = x + np.asarray(alibi, dtype=np.float64)[:, None, None] * rel[None]
    mask = causal_mask(seq_q, seq_kv, position_offset)
    if window > 0:
        mask = np.where(rel[None] <= -window, -np.inf, mask)
    s = x + mask
    mx = np.max(s, axis=-1, keepdims=True)
    if sinks is not None:
        snk = np.asarray(sinks, dtype=np.float64)[:, None, None]
        mx = np.maximum(mx, snk)
    e = np.exp(s - mx)
    den = np.sum(e, axis=-1, keepdims=True)
    if sinks is not None:
        den = den + np.exp(snk - mx)
    out = np.matmul(e / den, v_rep)
    return out.transpose(1, 0, 2)


def decode_arms(q, k, v, seq_lens, n_heads, n_kv_heads, scale, block_table=None, block_size=0,
                window=0, softcap=0.0, alibi=None, sinks=None, batch_indices=None):
    """Single-token decode with the arms of :func:`gqa_attention_arms`.

    Contiguous: ``k``/``v`` are ``[B, capacity, Hkv, D or Dv]``; paged: pools
    gathered through ``block_table``. The query of sequence ``b`` sits at
    position ``seq_lens[b] - 1`` (push-then-attend).
    """
    idx = range(q.shape[0]) if batch_indices is None else batch_indices
    out = []
    for b in idx:
        L = int(seq_lens[b])
        if block_table is None:
            kb, vb = k[b, :L], v[b, :L]
        else:
            kb = gather_paged(k, block_table[b], block_size, L)
            vb = gather_paged(v, block_table[b], block_size, L)
        out.append(gqa_attention_arms(q[b][None], kb, vb, n_heads, n_kv_heads, L - 1, scale,
                                      window, softcap, alibi, sinks)[0])
    return np.stack(out)


def gather_paged(pool: np.ndarray, block_table_row: np.ndarray, block_size: int,
                 seq_len: int) -> np.ndarray:
    """Rows ``0..seq_len`` of one sequence: token ``t`` is ``pool[bt[t // bs]][t % bs]``."""
    rows = []
    for t in range(seq_len):
        rows.append(pool[int(block_table_row[t // block_size]), t % block_size])
    if not rows:
        return np.zeros((0,) + pool.shape[2:], dtype=pool.dtype)
    return np.stack(rows, axis=0)


def prefill(q, k, v, n_heads, n_kv_heads, seq_kv, position_offset, scale,
            block_table=None, block_size=0, rows=None):
    """Batched causal prefill. ``q`` ``[B, seq_q, H, D]`` -> ``[B, seq_q, H, D]``.

    Contiguous: ``k``/``v`` are ``[B, capacity, Hkv, D]`` and the first
    ``seq_kv`` rows are used. Paged: ``k``/``v`` are pools and rows are
    gathered through ``block_table``. ``rows`` optionally restricts the
    computation to a list of query rows; each is the same definition with
    ``seq_q = 1`` at offset ``position_offset + i``.
    """
    B, seq_q = q.shape[0], q.shape[1]
    qsel = range(seq_q) if rows is None else rows
    out = np.zeros((B, len(qsel)) + q.shape[2:], dtype=np.float64)
    for b in range(B):
        if block_table is None:
            kb, vb = k[b, :seq_kv], v[b, :seq_kv]
        else:
            kb = gather_paged(k, block_table[b], block_size, seq_kv)
            vb = gather_paged(v, block_table[b], block_size, seq_kv)
        if rows is None:
            out[b] = gqa_attention(q[b], kb, vb, n_heads, n_kv_heads, position_offset, scale)
        else:
            for n, i in enumerate(qsel):
                out[b, n] = gqa_attention(q[b, i:i + 1], kb, vb, n_heads, n_kv_heads,
                                          position_offset + i, scale)[0]
    return out


def prefill_varlen(q, k, v, cu_q, seq_kv, n_heads, n_kv_heads, scale, block_table=None,
                   block_size=0, rows=None):
    """Causal prefill of a ragged batch: ``q`` packs every chunk ``[total_q, H, D]``.

    Sequence ``b`` owns query rows ``cu_q[b] .. cu_q[b+1]-1`` and holds
    ``seq_kv[b]`` keys (contiguous ``[B, capacity, Hkv, D]`` or gathered
    through ``block_table``); its chunk is the last ``n_b`` tokens, so its
    rows sit at offset ``seq_kv[b] - n_b``, and each sequence is the plain
    causal GQA of :func:`gqa_attention` on its own (the multi-sequence
    caller of frink-models 0.38.0 ``src/decoder/attn_block.rs``, ``KvStep``).
    ``rows`` optionally restricts the result to these packed rows.
    Returns ``[total_q, H, D]`` (or the selected rows).
    """
    total = int(cu_q[-1])
    want = range(total) if rows is None else rows
    pick = {r: n for n, r in enumerate(want)}
    out = np.zeros((len(pick),) + q.shape[1:], dtype=np.float64)
    for b in range(len(seq_kv)):
        s0, s1, L = int(cu_q[b]), int(cu_q[b + 1]), int(seq_kv[b])
        mine = [r for r in range(s0, s1) if r in pick]
        if not mine:
            continue
        if block_table is None:
            kb, vb = k[b, :L], v[b, :L]
        else:
            kb = gather_paged(k, block_table[b], block_size, L)
            vb = gather_paged(v, block_table[b], block_size, L)
        off = L - (s1 - s0)
        for r in mine:
            out[pick[r]] = gqa_attention(q[r:r + 1], kb, vb, n_heads, n_kv_heads, off + r - s0,
                                         scale)[0]
    return out


def decode_contig(q, k_cache, v_cache, seq_lens, n_heads, n_kv_heads, scale):
    """Single-token decode over a contiguous cache: ``q`` ``[B, H, D]`` -> ``[B, H, D]``.

    The query of sequence ``b`` sits at position ``seq_lens[b] - 1`` and its
    own key is already in the cache (push-then-attend).
    """
    B = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        out[b] = gqa_attention(q[b][None], k_cache[b, :L], v_cache[b, :L], n_heads,
                               n_kv_heads, L - 1, scale)[0]
    return out


def decode_paged(q, k_pool, v_pool, block_table, block_size, seq_lens, n_heads, n_kv_heads,
                 scale, batch_indices=None):
    """Single-token decode over a paged cache: gather through the block table, then decode."""
    idx = range(q.shape[0]) if batch_indices is None else batch_indices
    out = np.zeros((len(idx),) + q.shape[1:], dtype=np.float64)
    for n, b in enumerate(idx):
        L = int(seq_lens[b])
        kb = gather_paged(k_pool, block_table[b], block_size, L)
        vb = gather_paged(v_pool, block_table[b], block_size, L)
        out[n] = gqa_attention(q[b][None], kb, vb, n_heads, n_kv_heads, L - 1, scale)[0]
    return out


def mla_decode_latent(q_abs, latent, seq_lens, kv_lora_rank, scale, heads=None,
                      batch_indices=None):
    """Absorbed MLA decode over the latent cache.

    ``q_abs`` is ``[B, H, R + P]``, ``latent`` is ``[B, capacity, R + P]``.
    For each sequence and head: ``s_t = scale * q_abs[h] . latent[t]`` over
    the whole row, ``p = softmax(s)`` over ``t < seq_len``, and
    ``o_lat[h] = sum_t p_t * latent[t, :R]``. This is multi-query attention
    in which every head shares the latent as its key and its first ``R``
    entries as its value (frink-models 0.31.0 ``src/mla/mod.rs``,
    ``absorbed_attention``). Returns ``[B, H, R]`` (or the selected heads).
    """
    bidx = range(q_abs.shape[0]) if batch_indices is None else batch_indices
    hidx = range(q_abs.shape[1]) if heads is None else heads
    out = np.zeros((len(bidx), len(hidx), kv_lora_rank), dtype=np.float64)
    for n, b in enumerate(bidx):
        L = int(seq_lens[b])
        lat = np.asarray(latent[b, :L], dtype=np.float64)          # [L, R+P]
        qb = np.asarray(q_abs[b], dtype=np.float64)[list(hidx)]    # [h, R+P]
        # One shared KV head, every query head in its group (MQA).
        o = gqa_attention(qb[None], lat[:, None, :], lat[:, None, :kv_lora_rank],
                          len(hidx), 1, L - 1, scale)
        out[n] = o[0]
    return out


def mla_naive(q, c, k_rot, w_uk, w_uv, scale):
    """The naive MLA form for one sequence's last position, in float64.

    ``q`` is ``[H, qk_nope + qk_rope]`` (nope part first), ``c`` is
    ``[L, R]`` (normed latent per position), ``k_rot`` is ``[L, P]``
    (shared by every head), ``w_uk`` is ``[H, qk_nope, R]`` and ``w_uv`` is
    ``[H, v_dim, R]``. Each head's key per position is
    ``[w_uk[h] @ c_t | k_rot_t]`` and its value ``w_uv[h] @ c_t``; attention
    runs per head over every position (frink-models 0.31.0 ``src/mla/mod.rs``,
    ``naive_attention``). Returns ``[H, v_dim]``.
    """
    H = q.shape[0]
    L = c.shape[0]
    keys = np.concatenate([np.einsum("hnr,lr->lhn", w_uk, c),
                           np.broadcast_to(k_rot[:, None, :], (L, H, k_rot.shape[1]))], axis=2)
    vals = np.einsum("hvr,lr->lhv", w_uv, c)
    return gqa_attention(q[None], keys, vals, H, H, L - 1, scale)[0]


def mla_absorb_q(q, k_b):
    """The absorbed query: ``q_abs[.., h] = [k_b[h] @ q_nope[.., h] | q_rot[.., h]]``.

    ``q`` is ``[..., H, qk_nope + qk_rope]`` (nope part first), ``k_b`` is
    ``[H, R, qk_nope]``, one matrix per head in the absorb direction
    (frink-models 0.31.0 ``src/mla/mod.rs``: the ``MlaKvB::Split`` doc, and
    ``absorbed_attention``, which applies ``k_b[h]`` to the nope part and
    copies the rope part after it). Returns ``[..., H, R + qk_rope]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k_b = np.asarray(k_b, dtype=np.float64)
    nope = k_b.shape[2]
    absorbed = np.einsum("hrn,...hn->...hr", k_b, q[..., :nope])
    return np.concatenate([absorbed, q[..., nope:]], axis=-1)


def mla_up_proj(o_lat, v_b):
    """The per-head value up-projection: ``out[.., h] = v_b[h] @ o_lat[.., h]``.

    ``o_lat`` is ``[..., H, R]``, ``v_b`` is ``[H, v_head_dim, R]``
    (``MlaKvB::Split`` doc; the last loop of ``absorbed_attention``).
    Returns ``[..., H, v_head_dim]``.
    """
    return np.einsum("hvr,...hr->...hv", np.asarray(v_b, dtype=np.float64),
                     np.asarray(o_lat, dtype=np.float64))


def mla_absorbed(q, c, k_rot, w_uk, w_uv, scale):
    """The absorbed MLA form of :func:`mla_naive`: same result, latent-sized cache.

    The query's nope part is pulled through ``k_b[h] = w_uk[h]^T`` into latent
    space, attention runs over the cached latent rows ``[c_t | k_rot_t]`` with
    the first ``R`` entries as the value, and the weighted latent is pulled up
    through ``v_b[h] = w_uv[h]`` (frink-models 0.31.0 ``src/mla/mod.rs``,
    ``absorbed_attention``; the ``MlaKvB`` doc says the two forms compute
    the same attention).
    """
    R = c.shape[1]
    q_abs = mla_absorb_q(q, np.transpose(w_uk, (0, 2, 1)))
    latent = np.concatenate([c, k_rot], axis=1)
    o_lat = mla_decode_latent(q_abs[None], latent[None], [c.shape[0]], R, scale)[0]
    return mla_up_proj(o_lat, w_uv)


# ------------------------------------------------------------------ cache append (push)

def rope_interleaved(x, position, theta: float) -> np.ndarray:
    """Interleaved rotary embedding of the last axis of ``x`` at ``position``, in float64.

    The last axis (width ``d``, even) holds pairs ``(x[2i], x[2i+1])``; pair
    ``i`` turns by the angle ``position * theta ** (-2i / d)``:
    ``(a, b) -> (a cos - b sin, a sin + b cos)``. This is the rotation
    frink-models 0.31.0 ``src/mla/mod.rs`` applies to the shared ``k_rot``
    slice (module doc point 2, "interleaved convention"; ``rotate_pe`` with no
    YaRN factors). ``position`` broadcasts against ``x.shape[:-1]``.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("rotary width must be even")
    out = np.empty_like(x)
    pos = np.asarray(position, dtype=np.float64)
    for i in range(d // 2):
        angle = pos * float(theta) ** (-2.0 * i / d)
        c, s = np.cos(angle), np.sin(angle)
        a, b = x[..., 2 * i], x[..., 2 * i + 1]
        out[..., 2 * i] = a * c - b * s
        out[..., 2 * i + 1] = a * s + b * c
    return out


def append_rows(cache, new_rows, positions, block_table=None, block_size=0):
    """Push ``n_new`` rows per sequence into a KV cache; returns the updated copy.

    ``new_rows`` is ``[B, n_new, ...]``; row ``i`` of sequence ``b`` becomes
    token ``t = positions[b] + i`` of that sequence (``positions[b]`` = rows it
    held before the push). Contiguous (``block_table is None``): ``cache`` is
    ``[B, capacity, ...]`` and the row lands at ``cache[b, t]``. Paged:
    ``cache`` is a pool ``[num_blocks, block_size, ...]`` and the row lands at
    ``pool[block_table[b][t // block_size]][t % block_size]``. Push-then-attend:
    frink-models 0.38.0 ``src/decoder/attn_block.rs`` (``push_and_attend_row``
    writes this row to whichever backing, then attends); kopitiam-runtime 0.2.4
    ``src/attention.rs`` (``attention_forward`` appends before scoring).
    """
    out = np.array(cache, copy=True)
    B, n_new = new_rows.shape[0], new_rows.shape[1]
    for b in range(B):
        for i in range(n_new):
            t = int(positions[b]) + i
            if block_table is None:
                out[b, t] = new_rows[b, i]
            else:
                out[int(block_table[b][t // block_size]), t % block_size] = new_rows[b, i]
    return out


def mla_append_latent(latent, c_new, k_rot_new, positions, theta, block_table=None,
                      block_size=0):
    """Push one latent row ``[c | rope(k_rot)]`` per sequence; returns the updated float64 copy.

    ``c_new`` is ``[B, R]`` (the normed compressed KV), ``k_rot_new`` is
    ``[B, P]`` before rotation; the row written at token ``positions[b]`` is
    ``c_new[b]`` followed by ``k_rot_new[b]`` turned by :func:`rope_interleaved`
    at that position, once, for every head to share. ``theta <= 0`` means no
    rotation (the rope-free configuration). frink-models 0.31.0
    ``src/mla/mod.rs``: ``mla_forward_token`` (``k_rot`` rotated once before
    broadcasting) and ``absorbed_attention`` (``k_cache`` extended by ``c``
    then ``k_rot``). Layout as :func:`append_rows` with one row per sequence.
    """
    c_new = np.asarray(c_new, dtype=np.float64)
    k_rot = np.asarray(k_rot_new, dtype=np.float64)
    if theta > 0:
        k_rot = rope_interleaved(k_rot, np.asarray(positions, dtype=np.float64), theta)
    rows = np.concatenate([c_new, k_rot], axis=-1)[:, None, :]
    return append_rows(np.asarray(latent, dtype=np.float64), rows, positions, block_table,
                       block_size)
