"""GPU parity where the running max must move mid-sequence.

Every kernel keeps a reference max per row (head) and rescales O and l only
when a later key's score beats it by more than 2^8 in the exp2 domain. With
iid inputs of order 1 that never happens after the first tile, so these
cases scale the keys by a factor that grows with the key position (and add
a few isolated large keys): later tiles then beat the reference by far, many
times per row. Only keys are scaled, so outputs stay of order 1 and the
usual tolerances apply. Each test first checks, on the inputs, that the
rescale condition does occur.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_causal_amd as pk
from oracle import oracle as O
from paged_kv_attention_causal_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"f32": 2e-3, "bf16": 2e-2}
LOG2E = 1.4426950408889634


def dev(a, dtype="bf16"):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).to(DEV)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)


def check(got, ref, dtype, what):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    say(f"  {what}: max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
    assert err.max() <= TOL[dtype], f"{what}: {err.max():.3e}"


def as_dtype(a, dtype="bf16"):
    """The values the kernel will see: a scaled bf16 input is rounded to bf16 again
    (to nearest even) before both the kernel and the oracle read it."""
    if dtype != "bf16":
        return a
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def growth(n, top, spikes=()):
    """Per-position key factor: 1 at position 0 rising linearly to ``top``, and
    4 x that at the ``spikes`` positions."""
    f = 1.0 + (top - 1.0) * np.arange(n) / max(1, n - 1)
    for j in spikes:
        if j < n:
            f[j] *= 4.0
    return f


def assert_max_moves(q, k, c, tile, lo=1):
    """The inputs make the kernels' lazy rescale fire: for at least one row, a
    key tile after the first beats the first tile's max by > 8 (exp2 domain).
    q [R, D], k [L, D] of one head; c = scale * log2(e)."""
    s = (q.astype(np.float64) @ k.astype(np.float64).T) * c
    first = s[:, :tile].max(axis=1)
    later = s[:, tile:].max(axis=1) if s.shape[1] > tile else first
    moved = int(np.sum(later - first > 8.0))
    assert moved >= lo, "the test inputs do not move the running max"
    return moved


def scale_pool_rows(pool, block_table, lens, bs, f_of_len):
    """Multiply the pool row of position j of sequence b by f_of_len(L_b)[j]."""
    out = pool.copy()
    for b, L in enumerate(lens):
        L = int(L)
        f = f_of_len(L)
        j = np.arange(L)
        blk = block_table[b, j // bs]
        out[blk, j % bs] *= f.reshape((-1,) + (1,) * (pool.ndim - 2)).astype(out.dtype)
    return out


@pytest.mark.parametrize("dtype,D,paged,top", [("bf16", 128, False, 9.0), ("bf16", 128, True, 9.0),
                                               ("f32", 16, False, 40.0)])
def test_prefill_running_max_moves(dtype, D, paged, top):
    B, H, Hkv, sq, off = 2, 4, 2, 300, 260
    say(f"case: prefill with growing keys dtype={dtype} D={D} paged={paged} top={top}")
    c = inputs.prefill_case(17, dtype=dtype, batch=B, n_heads=H, n_kv_heads=Hkv, head_dim=D,
                            seq_q=sq, position_offset=off, scale=0.25 if dtype == "f32" else None)
    L = off + sq
    f = growth(L, top, spikes=(150, 333, 470))
    k = as_dtype((c.k * f[None, :, None, None]).astype(np.float32), dtype)
    moved = assert_max_moves(c.q[0, -32:, 0], k[0, :, 0], c.scale * LOG2E, 64)   # rows that see every key
    say(f"  rows whose max moves after the first tile (b0, h0): {moved}")
    ref = O.prefill(c.q, k, c.v, H, Hkv, L, off, c.scale)
    if paged:
        bs = 16
        rng = np.random.default_rng(4)
        nb = (L + bs - 1) // bs
        perm = rng.permutation(B * nb + 3)
        bt = perm[:B * nb].reshape(B, nb).astype(np.int32)
        kp = np.full((B * nb + 3, bs, Hkv, D), np.nan, np.float32)
        vp = np.full_like(kp, np.nan)
        for b in range(B):
            for i in range(nb):
                rows = slice(i * bs, min(L, (i + 1) * bs))
                n = rows.stop - rows.start
                kp[bt[b, i], :n] = k[b, rows]
                vp[bt[b, i], :n] = c.v[b, rows]
        o = pk.attn_prefill(dev(c.q, dtype), dev(kp, dtype), dev(vp, dtype), seq_kv=L,
                            position_offset=off, attention_scale=c.scale, block_table=i32(bt))
    else:
        o = pk.attn_prefill(dev(c.q, dtype), dev(k, dtype), dev(c.v, dtype), seq_kv=L,
                            position_offset=off, attention_scale=c.scale)
    check(host(o), ref, dtype, "prefill, growing keys")


def test_varlen_running_max_moves():
    say("case: ragged prefill with growing keys")
    q_lens, cached = [90, 300, 1, 257], [400, 0, 700, 33]
    c = inputs.varlen_prefill_case(23, q_lens=q_lens, cached=cached, n_heads=4, n_kv_heads=2,
                                   block_size=16)
    k = as_dtype(scale_pool_rows(c.k, c.block_table, c.seq_kv, 16,
                                 lambda L: growth(L, 9.0, (200, 500))))
    b = 0
    L0 = int(c.seq_kv[b])
    kb = np.stack([k[c.block_table[b, j // 16], j % 16, 0] for j in range(L0)])
    assert_max_moves(c.q[int(c.cu_q[b]):int(c.cu_q[b + 1]), 0], kb, c.scale * LOG2E, 64)
    o = pk.attn_prefill_varlen(dev(c.q), dev(k), dev(c.v), i32(c.cu_q), i32(c.seq_kv),
                               max_seq_q=max(q_lens), attention_scale=c.scale,
                               block_table=i32(c.block_table))
    ref = O.prefill_varlen(c.q, k, c.v, c.cu_q, c.seq_kv, 4, 2, c.scale, c.block_table, 16)
    check(host(o), ref, "bf16", "ragged prefill, growing keys")


@pytest.mark.parametrize("dtype,D,top", [("bf16", 128, 9.0), ("f32", 16, 40.0)])
def test_decode_running_max_moves(dtype, D, top):
    lens = [3000, 700, 65, 1500]
    say(f"case: decode with growing keys dtype={dtype} D={D} lens={lens}")
    c = inputs.paged_decode_case(29, dtype=dtype, batch=len(lens), n_heads=8, n_kv_heads=2,
                                 head_dim=D, block_size=16, seq_lens=lens, len_hi=3000,
                                 scale=0.3 if dtype == "f32" else None)
    kp = as_dtype(scale_pool_rows(c.k_pool, c.block_table, lens, 16,
                                  lambda L: growth(L, top, (L // 3, (2 * L) // 3))), dtype)
    k0 = np.stack([kp[c.block_table[0, j // 16], j % 16, 0] for j in range(lens[0])])
    assert_max_moves(c.q[0, :4], k0, c.scale * LOG2E, 64)
    maxlen = int(c.block_table.shape[1] * 16)
    o = pk.attn_decode_paged(dev(c.q, dtype), dev(kp, dtype), dev(c.v_pool, dtype),
                             i32(c.block_table), i32(c.seq_lens), max_seq_len=maxlen,
                             attention_scale=c.scale)
    ref = O.decode_paged(c.q, kp, c.v_pool, c.block_table, 16, c.seq_lens, 8, 2, c.scale)
    check(host(o), ref, dtype, "paged decode, growing keys")
    # the same rows laid out contiguously: bitwise the paged result
    kc = np.full((len(lens), maxlen, 2, D), np.nan, np.float32)
    vc = np.full_like(kc, np.nan)
    for b, L in enumerate(lens):
        j = np.arange(L)
        kc[b, :L] = kp[c.block_table[b, j // 16], j % 16]
        vc[b, :L] = c.v_pool[c.block_table[b, j // 16], j % 16]
    oc = pk.attn_decode_contig(dev(c.q, dtype), dev(kc, dtype), dev(vc, dtype), i32(c.seq_lens),
                               max_seq_len=maxlen, attention_scale=c.scale)
    assert torch.equal(oc, o), "contiguous != paged (bitwise)"


def test_mla_running_max_moves():
    lens = [1800, 300, 64]
    say(f"case: MLA with growing rope keys, lens={lens}")
    cap = max(lens) + 4
    c = inputs.mla_case(31, batch=len(lens), ctx=cap, seq_lens=lens, n_heads=64)
    lat = c.latent.copy()
    f = growth(cap, 25.0, (100, 900))
    lat[:, :, 512:] *= f[None, :, None].astype(lat.dtype)   # k_rot only: values stay of order 1
    lat = as_dtype(lat)
    assert_max_moves(c.q_abs[0], lat[0, :lens[0]], c.scale * LOG2E, 32)
    ref = O.mla_decode_latent(c.q_abs, lat, lens, 512, c.scale)
    poisoned = lat.copy()
    for b, L in enumerate(lens):
        poisoned[b, L:] = np.nan
    o = pk.mla_decode_latent(dev(c.q_abs), dev(poisoned), i32(lens), kv_lora_rank=512,
                             max_seq_len=max(lens), attention_scale=c.scale)
    check(host(o), ref, "bf16", "MLA, growing rope keys")
    # paged latent pool, blocks of 16 rows dealt at random: bitwise the contiguous result
    bs = 16
    nb = (cap + bs - 1) // bs
    rng = np.random.default_rng(6)
    perm = rng.permutation(len(lens) * nb + 5)
    bt = perm[:len(lens) * nb].reshape(len(lens), nb).astype(np.int32)
    pool = np.full((len(lens) * nb + 5, bs, 576), np.nan, np.float32)
    for b in range(len(lens)):
        for i in range(nb):
            rows = slice(i * bs, min(cap, (i + 1) * bs))
            pool[bt[b, i], :rows.stop - rows.start] = poisoned[b, rows]
    op = pk.mla_decode_latent_paged(dev(c.q_abs), dev(pool), i32(bt), i32(lens),
                                    kv_lora_rank=512, max_seq_len=max(lens),
                                    attention_scale=c.scale)
    assert torch.equal(op, o), "paged latent != contiguous latent (bitwise)"


def test_decode_arms_running_max_moves():
    lens = [2500, 400, 1200]
    H, Hkv, D = 8, 2, 128
    say(f"case: decode with arms (ALiBi, sinks, window) and growing keys, lens={lens}")
    c = inputs.paged_decode_case(37, batch=len(lens), n_heads=H, n_kv_heads=Hkv, head_dim=D,
                                 block_size=16, seq_lens=lens, len_hi=2560)
    kp = as_dtype(scale_pool_rows(c.k_pool, c.block_table, lens, 16,
                                  lambda L: growth(L, 9.0, (L // 4, L // 2))))
    k0 = np.stack([kp[c.block_table[0, j // 16], j % 16, 0] for j in range(lens[0])])
    assert_max_moves(c.q[0, :4], k0, c.scale * LOG2E, 64)
    maxlen = int(c.block_table.shape[1] * 16)
    kc = np.full((len(lens), maxlen, Hkv, D), np.nan, np.float32)
    vc = np.full_like(kc, np.nan)
    for b, L in enumerate(lens):
        j = np.arange(L)
        kc[b, :L] = kp[c.block_table[b, j // 16], j % 16]
        vc[b, :L] = c.v_pool[c.block_table[b, j // 16], j % 16]
    alibi = inputs.alibi_slopes(H)
    sinks = inputs.sink_logits(5, H)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    kw = dict(max_seq_len=maxlen, attention_scale=c.scale, window=2000, alibi=f32(alibi),
              sinks=f32(sinks))
    op = pk.attn_decode_paged_ext(dev(c.q), dev(kp), dev(c.v_pool), i32(c.block_table),
                                  i32(c.seq_lens), **kw)
    oc = pk.attn_decode_contig_ext(dev(c.q), dev(kc), dev(vc), i32(c.seq_lens), **kw)
    assert torch.equal(op, oc), "contiguous != paged (bitwise)"
    ref = O.decode_arms(c.q, kc, vc, c.seq_lens, H, Hkv, c.scale, window=2000, softcap=0.0,
                        alibi=alibi, sinks=sinks)
    check(host(op), ref, "bf16", "decode arms, growing keys")
