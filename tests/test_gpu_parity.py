"""GPU parity: the HIP kernels (through the C-ABI) against the float64 oracle.

Both sides read the same seeded inputs (paged_kv_attention_causal_amd.inputs).
Tolerances: max |err| <= 2e-3 for fp32 I/O and <= 2e-2 for bf16 I/O, against
oracle values of order 1; stricter diagnostics (err / output RMS) are printed.
Paged and contiguous decode of the same rows must agree bitwise; so must two
runs of the same call. Rows a call must not read are poisoned with NaN.
"""
import math

import numpy as np
import pytest
import torch

import paged_kv_attention_causal_amd as pk
from oracle import oracle as O
from paged_kv_attention_causal_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"f32": 2e-3, "bf16": 2e-2}


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(_tdt(dtype)).to(DEV)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)


def check(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) or 1.0
    say(f"  {what}: max|err|={err.max():.3e} mean|err|={err.mean():.3e} "
        f"max|err|/rms={err.max() / rms:.3e} rms={rms:.3e}")
    assert err.max() <= TOL[dtype], f"{what}: max abs error {err.max():.3e} > {TOL[dtype]}"
    return err.max()


def pool_from_contig(kc, vc, lens, bs, rng, slack_fill=np.nan):
    """Scatter contiguous [B, cap, Hkv, D] rows into a shuffled pool of bs-row blocks."""
    B = kc.shape[0]
    need = [(int(L) + bs - 1) // bs for L in lens]
    nb = sum(need) + 3
    perm = rng.permutation(nb)
    maxb = max(need)
    bt = np.full((B, maxb), -1, dtype=np.int32)
    kp = np.full((nb, bs) + kc.shape[2:], slack_fill, dtype=np.float32)
    vp = np.full((nb, bs) + kc.shape[2:], slack_fill, dtype=np.float32)
    o = 0
    for b in range(B):
        L = int(lens[b])
        for j in range(need[b]):
            blk = perm[o]
            o += 1
            bt[b, j] = blk
            n = min(bs, L - j * bs)
            kp[blk, :n] = kc[b, j * bs:j * bs + n]
            vp[blk, :n] = vc[b, j * bs:j * bs + n]
    return kp, vp, bt


# ------------------------------------------------------------------ tiny fp32

def test_tiny_f32_prefill_then_decode_steps():
    say("case: tiny fp32 H=4 Hkv=2 D=16, prefill 64 then 8 decode steps")
    q, k, v, scale = inputs.tiny_f32(0)
    H, Hkv, D = 4, 2, 16
    # prefill over the first 64 rows; rows 64.. of the cache are poison
    kc = k.copy()
    vc = v.copy()
    kc[:, 64:] = np.nan
    vc[:, 64:] = np.nan
    o = pk.attn_prefill(dev(q[:, :64], "f32"), dev(kc, "f32"), dev(vc, "f32"), seq_kv=64,
                        position_offset=0, attention_scale=scale)
    ref = O.prefill(q[:, :64], k, v, H, Hkv, 64, 0, scale)
    check(host(o), ref, "f32", "prefill 64")
    full = O.prefill(q, k, v, H, Hkv, 72, 0, scale)
    rng = np.random.default_rng(5)
    for s in range(8):
        L = 65 + s
        kc = k.copy()
        vc = v.copy()
        kc[:, L:] = np.nan
        vc[:, L:] = np.nan
        qd = dev(q[:, 64 + s], "f32")
        lens = i32([L])
        oc = pk.attn_decode_contig(qd, dev(kc, "f32"), dev(vc, "f32"), lens, max_seq_len=L,
                                   attention_scale=scale)
        ref = O.decode_contig(q[:, 64 + s], k, v, [L], H, Hkv, scale)
        check(host(oc), ref, "f32", f"decode step {s} (L={L})")
        # decode step s equals row 64+s of a prefill over the whole sequence
        check(host(oc), full[:, 64 + s], "f32", f"decode step {s} vs prefill row")
        kp, vp, bt = pool_from_contig(kc, vc, [L], 16, rng)
        op = pk.attn_decode_paged(qd, dev(kp, "f32"), dev(vp, "f32"), i32(bt), lens,
                                  max_seq_len=L, attention_scale=scale)
        assert torch.equal(op, oc), f"paged != contiguous at step {s}"


# ------------------------------------------------------------------ prefill

PREFILL_CASES = [
    # (B, H, Hkv, D, seq_q, off, extra_kv, paged_bs, dtype, scale)
    (2, 8, 2, 128, 300, 0, 0, 0, "bf16", None),
    (2, 8, 8, 128, 200, 77, 0, 0, "bf16", None),
    (1, 16, 2, 128, 129, 500, 0, 16, "bf16", None),
    (3, 4, 4, 128, 1, 999, 0, 1, "bf16", None),
    (1, 7, 1, 128, 65, 63, 0, 64, "bf16", 0.05),
    (2, 4, 2, 128, 50, 10, 140, 0, "bf16", None),     # seq_kv beyond off + seq_q
    (2, 4, 2, 128, 50, 10, 140, 16, "bf16", None),
    (1, 4, 2, 16, 77, 5, 0, 0, "f32", 0.25),
    (2, 6, 3, 16, 130, 0, 0, 4, "f32", 0.7),
    (1, 2, 1, 128, 40, 0, 0, 0, "bf16", 0.0),         # scale 0: uniform weights
    # chunks no longer than their history: items grouped by KV head, with a
    # whole XCD run plus a tail, and an all-tail grid
    (5, 6, 3, 128, 300, 400, 0, 16, "bf16", None),
    (3, 8, 2, 128, 513, 600, 0, 0, "bf16", None),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "B{}H{}Hkv{}D{}q{}off{}x{}bs{}{}".format(*c[:9]))
def test_prefill_small(case):
    B, H, Hkv, D, sq, off, extra, bs, dtype, scale = case
    say(f"case: prefill {case}")
    c = inputs.prefill_case(11, dtype=dtype, batch=B, n_heads=H, n_kv_heads=Hkv, head_dim=D,
                            seq_q=sq, position_offset=off, scale=scale,
                            kv_capacity=off + sq + extra + 5)
    seq_kv = off + sq + extra
    kc, vc = c.k.copy(), c.v.copy()
    kc[:, seq_kv:] = np.nan
    vc[:, seq_kv:] = np.nan
    ref = O.prefill(c.q, c.k, c.v, H, Hkv, seq_kv, off, c.scale)
    if bs:
        kp, vp, bt = pool_from_contig(kc, vc, [seq_kv] * B, bs, np.random.default_rng(3))
        o = pk.attn_prefill(dev(c.q, dtype), dev(kp, dtype), dev(vp, dtype), seq_kv=seq_kv,
                            position_offset=off, attention_scale=c.scale, block_table=i32(bt))
    else:
        o = pk.attn_prefill(dev(c.q, dtype), dev(kc, dtype), dev(vc, dtype), seq_kv=seq_kv,
                            position_offset=off, attention_scale=c.scale)
    check(host(o), ref, dtype, "prefill")
    if off == 0 and extra == 0:
        # row 0 sees key 0 only: exactly v[0] of its KV head on the GPU too
        o0 = host(o)[:, 0]
        for h in range(H):
            assert np.array_equal(o0[:, h], c.v[:, 0, h // (H // Hkv)].astype(np.float64))


@pytest.fixture(scope="module")
def prefill_full():
    say("generating causal prefill bf16 B=1 H=28 Hkv=4 D=128 S=4096")
    return inputs.prefill_case(0)


def test_prefill_full_size_sampled_rows(prefill_full):
    c = prefill_full
    say("case: causal prefill bf16 full size (sampled rows)")
    q, k, v = dev(c.q, "bf16"), dev(c.k, "bf16"), dev(c.v, "bf16")
    o = pk.attn_prefill(q, k, v, seq_kv=c.seq_kv, position_offset=0, attention_scale=c.scale)
    o2 = pk.attn_prefill(q, k, v, seq_kv=c.seq_kv, position_offset=0, attention_scale=c.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2), "prefill is not deterministic"
    rng = np.random.default_rng(1)
    # the first and last row of every 256-row query tile (each tile and head is
    # its own work item), the rows around the first key tiles, and a random draw
    edges = [r for t in range(16) for r in (256 * t, 256 * t + 255)]
    rows = sorted(set(edges + [1, 31, 32, 63, 64, 127, 128, 129, 4000, 4094]
                      + rng.integers(0, 4096, 18).tolist()))
    ref = O.prefill(c.q, c.k, c.v, 28, 4, c.seq_kv, 0, c.scale, rows=rows)
    check(host(o)[:, rows], ref, "bf16", "prefill 4096 sampled rows")


def test_chunked_paged_prefill_full_size_sampled_rows():
    say("case: chunked prefill on paged KV bf16 full size (sampled rows)")
    c = inputs.chunked_paged_prefill_case(0)
    o = pk.attn_prefill(dev(c.q, "bf16"), dev(c.k, "bf16"), dev(c.v, "bf16"), seq_kv=c.seq_kv,
                        position_offset=c.position_offset, attention_scale=c.scale,
                        block_table=i32(c.block_table))
    oh = host(o)
    rng = np.random.default_rng(2)
    rows = sorted(set([0, 1, 127, 128, 255, 256, 511] + rng.integers(0, 512, 6).tolist()))
    for b in range(c.batch):
        ref = O.prefill(c.q[b:b + 1], c.k, c.v, 32, 8, c.seq_kv, c.position_offset, c.scale,
                        block_table=c.block_table[b:b + 1], block_size=16, rows=rows)
        check(oh[b:b + 1, rows], ref, "bf16", f"seq {b}")


def test_prefill_bad_block_id_gives_nan_rows():
    say("case: prefill with an out-of-pool block id")
    c = inputs.chunked_paged_prefill_case(4, batch=2, cached=40, seq_q=30, n_heads=4,
                                          n_kv_heads=2, head_dim=128, block_size=16)
    bt = c.block_table.copy()
    bt[1, 2] = c.k.shape[0] + 7      # sequence 1 names a block past the pool
    o = host(pk.attn_prefill(dev(c.q, "bf16"), dev(c.k, "bf16"), dev(c.v, "bf16"),
                             seq_kv=c.seq_kv, position_offset=40, attention_scale=c.scale,
                             block_table=i32(bt)))
    assert np.all(np.isnan(o[1]))
    ref = O.prefill(c.q[:1], c.k, c.v, 4, 2, c.seq_kv, 40, c.scale, block_table=c.block_table[:1],
                    block_size=16)
    check(o[:1], ref, "bf16", "clean sequence")


# ------------------------------------------------------------------ decode

@pytest.fixture(scope="module")
def decode_full():
    say("generating paged decode bf16 64 seqs L~U[512,8192] H=32 Hkv=8 D=128 bs=16")
    return inputs.paged_decode_case(0)


def _run_paged(c, kp=None, vp=None, bt=None, lens=None):
    kp = dev(c.k_pool, c.dtype) if kp is None else kp
    vp = dev(c.v_pool, c.dtype) if vp is None else vp
    bt = i32(c.block_table) if bt is None else bt
    lens = i32(c.seq_lens) if lens is None else lens
    return pk.attn_decode_paged(dev(c.q, c.dtype), kp, vp, bt, lens,
                                max_seq_len=int(c.block_table.shape[1] * c.block_size),
                                attention_scale=c.scale)


def test_paged_decode_full_size(decode_full):
    c = decode_full
    say(f"case: paged decode full size, sum L = {int(c.seq_lens.sum())}, pool {c.k_pool.shape[0]} blocks")
    kp, vp = dev(c.k_pool, "bf16"), dev(c.v_pool, "bf16")
    bt, lens = i32(c.block_table), i32(c.seq_lens)
    o = _run_paged(c, kp, vp, bt, lens)
    o2 = _run_paged(c, kp, vp, bt, lens)
    assert torch.equal(o, o2), "paged decode is not deterministic"
    ref = O.decode_paged(c.q, c.k_pool, c.v_pool, c.block_table, 16, c.seq_lens, 32, 8, c.scale)
    check(host(o), ref, "bf16", "paged decode, all 64 sequences")
    # Contiguous cache holding the same rows (NaN past each length): bitwise equal.
    cap = 8192
    kc = torch.full((64, cap, 8, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, float("nan"))
    btl = bt.long()
    for b in range(64):
        L = int(c.seq_lens[b])
        nb = (L + 15) // 16
        kc[b, :L] = kp[btl[b, :nb]].reshape(nb * 16, 8, 128)[:L]
        vc[b, :L] = vp[btl[b, :nb]].reshape(nb * 16, 8, 128)[:L]
    oc = pk.attn_decode_contig(dev(c.q, "bf16"), kc, vc, lens, max_seq_len=cap,
                               attention_scale=c.scale)
    assert torch.equal(oc, o), "contiguous != paged (bitwise)"
    del kc, vc
    # Poison every pool row no sequence reads: the result must not move.
    used = np.zeros((c.k_pool.shape[0], 16), dtype=bool)
    for b in range(64):
        L = int(c.seq_lens[b])
        for t in range(0, L, 16):
            used[c.block_table[b, t // 16], :min(16, L - t)] = True
    mask = torch.from_numpy(~used).to(DEV)
    kp[mask] = float("nan")
    vp[mask] = float("nan")
    o3 = _run_paged(c, kp, vp, bt, lens)
    assert torch.equal(o3, o), "output changed when unread rows were poisoned"


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 16)])
@pytest.mark.parametrize("H,Hkv", [(8, 8), (8, 4), (16, 4), (16, 2), (6, 2), (7, 1), (3, 3)])
@pytest.mark.parametrize("bs", [1, 16, 256])
def test_decode_edge_lengths(dtype, D, H, Hkv, bs):
    lens = [1, 2, 255, 256, 257, 511, 512, 513, 700]
    say(f"case: decode edges dtype={dtype} D={D} H={H} Hkv={Hkv} bs={bs} lens={lens}")
    c = inputs.paged_decode_case(21, dtype=dtype, batch=len(lens), n_heads=H, n_kv_heads=Hkv,
                                 head_dim=D, block_size=bs, seq_lens=lens, len_hi=768,
                                 scale=0.3 if dtype == "f32" else None)
    o = _run_paged(c)
    ref = O.decode_paged(c.q, c.k_pool, c.v_pool, c.block_table, bs, c.seq_lens, H, Hkv, c.scale)
    check(host(o), ref, dtype, "paged")
    kc, vc = c.contig(capacity=768, fill=np.nan)
    oc = pk.attn_decode_contig(dev(c.q, dtype), dev(kc, dtype), dev(vc, dtype), i32(c.seq_lens),
                               max_seq_len=768, attention_scale=c.scale)
    assert torch.equal(oc, o), "contiguous != paged (bitwise)"
    # length 1: the query sees only its own key -> exactly v[0] of the KV head
    oh = host(o)
    for h in range(H):
        assert np.array_equal(oh[0, h], vc[0, 0, h // (H // Hkv)].astype(np.float64))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 16)])
def test_decode_zero_scale_is_the_mean_of_the_visible_values(dtype, D):
    lens = [1, 70, 513, 1000]
    say(f"case: decode at attention_scale 0, dtype={dtype}, lens={lens}")
    c = inputs.paged_decode_case(13, dtype=dtype, batch=len(lens), n_heads=8, n_kv_heads=2,
                                 head_dim=D, block_size=16, seq_lens=lens, len_hi=1024, scale=0.0)
    o = _run_paged(c)
    ref = O.decode_paged(c.q, c.k_pool, c.v_pool, c.block_table, 16, c.seq_lens, 8, 2, 0.0)
    # the oracle at scale 0 is the plain mean of the visible V rows
    kc, vc = c.contig(capacity=1024, fill=np.nan)
    for b, L in enumerate(lens):
        mean = vc[b, :L].astype(np.float64).mean(axis=0)          # [Hkv, D]
        assert np.allclose(ref[b], np.repeat(mean, 4, axis=0), atol=1e-12)
    check(host(o), ref, dtype, "paged, scale 0")
    oc = pk.attn_decode_contig(dev(c.q, dtype), dev(kc, dtype), dev(vc, dtype), i32(c.seq_lens),
                               max_seq_len=1024, attention_scale=0.0)
    assert torch.equal(oc, o), "contiguous != paged (bitwise) at scale 0"


@pytest.mark.parametrize("H,bs,B,lo,maxlen", [(4, 1, 256, 3000, 8192), (8, 2, 512, 1000, 8200)])
def test_paged_decode_wide_block_windows(H, bs, B, lo, maxlen):
    """Pieces longer than the 1023-block LDS window (tiny blocks, long contexts):
    the kernel walks sub-pieces; it must match the oracle and stay bitwise equal to
    the contiguous kernel, which takes each piece in one pass."""
    say(f"case: paged decode with sub-pieces, B={B} H={H} Hkv=1 bs={bs} lens U[{lo},{maxlen}]")
    c = inputs.paged_decode_case(17, batch=B, len_lo=lo, len_hi=maxlen, n_heads=H,
                                 n_kv_heads=1, head_dim=128, block_size=bs)
    # the launcher takes the sub-piece kernel whenever B * max_seq_len / ranges
    # needs more than 1022 block ids, and at most 2048 ranges are cut
    assert B * maxlen // bs > 1022 * 2048
    kp, vp = dev(c.k_pool, "bf16"), dev(c.v_pool, "bf16")
    bt, lens = i32(c.block_table), i32(c.seq_lens)
    o = _run_paged(c, kp, vp, bt, lens)
    sel = [0, 1, 77, 128, 200, B - 1]
    ref = O.decode_paged(c.q, c.k_pool, c.v_pool, c.block_table, bs, c.seq_lens, H, 1, c.scale,
                         batch_indices=sel)
    check(host(o)[sel], ref, "bf16", f"sequences {sel}")
    kc = torch.full((B, maxlen, 1, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, float("nan"))
    btl = bt.long()
    for b in range(B):
        L = int(c.seq_lens[b])
        nb = (L + bs - 1) // bs
        kc[b, :L] = kp[btl[b, :nb]].reshape(nb * bs, 1, 128)[:L]
        vc[b, :L] = vp[btl[b, :nb]].reshape(nb * bs, 1, 128)[:L]
    oc = pk.attn_decode_contig(dev(c.q, "bf16"), kc, vc, lens, max_seq_len=maxlen,
                               attention_scale=c.scale)
    assert torch.equal(oc, o), "contiguous != paged (bitwise) with sub-pieces"


def test_decode_bad_entries_give_nan_only_there():
    say("case: decode with a zero length and an out-of-pool block id")
    c = inputs.paged_decode_case(8, batch=5, len_lo=100, len_hi=600, n_heads=8, n_kv_heads=2)
    clean = host(_run_paged(c))
    lens = c.seq_lens.copy()
    lens[1] = 0
    bt = c.block_table.copy()
    bt[3, 1] = -5
    o = host(_run_paged(c, bt=i32(bt), lens=i32(lens)))
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(o[3]))
    # The other sequences stay correct. (The token ranges are cut over the valid
    # lengths, so their rounding may differ from the clean run's.)
    keep = [0, 2, 4]
    ref = O.decode_paged(c.q, c.k_pool, c.v_pool, c.block_table, 16, c.seq_lens, 8, 2, c.scale,
                         batch_indices=keep)
    check(o[keep], ref, "bf16", "untouched sequences")
    check(clean[keep], ref, "bf16", "clean run")


# ------------------------------------------------------------------ MLA

def test_mla_full_size_sampled_sequences():
    say("case: MLA latent decode bf16 B=32 ctx=4096 H=128 R=512 P=64")
    c = inputs.mla_case(0)
    q, lat, lens = dev(c.q_abs, "bf16"), dev(c.latent, "bf16"), i32(c.seq_lens)
    o = pk.mla_decode_latent(q, lat, lens, kv_lora_rank=512, max_seq_len=4096,
                             attention_scale=c.scale)
    o2 = pk.mla_decode_latent(q, lat, lens, kv_lora_rank=512, max_seq_len=4096,
                              attention_scale=c.scale)
    assert torch.equal(o, o2), "MLA decode is not deterministic"
    oh = host(o)
    bsel = [0, 7, 13, 31]
    ref = O.mla_decode_latent(c.q_abs, c.latent, c.seq_lens, 512, c.scale, batch_indices=bsel)
    check(oh[bsel], ref, "bf16", "MLA sequences 0,7,13,31, all heads")
    # Every sequence (each one is eight context pieces, one workgroup each),
    # eight heads spread over the four 32-head waves.
    heads = [0, 17, 33, 50, 64, 95, 100, 127]
    ref = O.mla_decode_latent(c.q_abs, c.latent, c.seq_lens, 512, c.scale, heads=heads)
    check(oh[:, heads], ref, "bf16", "MLA all 32 sequences, 8 heads")


@pytest.mark.parametrize("lens", [[1000, 37], [1, 64, 65, 129], [4096]])
def test_mla_split_context(lens):
    say(f"case: MLA with a split context, lens={lens}")
    cap = max(lens) + 3
    c = inputs.mla_case(3, batch=len(lens), ctx=cap, seq_lens=lens)
    lat = c.latent.copy()
    for b, L in enumerate(lens):
        lat[b, L:] = np.nan
    o = pk.mla_decode_latent(dev(c.q_abs, "bf16"), dev(lat, "bf16"), i32(lens),
                             kv_lora_rank=512, max_seq_len=max(lens), attention_scale=c.scale)
    ref = O.mla_decode_latent(c.q_abs, c.latent, lens, 512, c.scale)
    check(host(o), ref, "bf16", "MLA split")


@pytest.mark.parametrize("n_heads,batch,lens", [
    (8, 2, [64, 5]),               # fewer heads than one wave's 32
    (16, 3, [200, 31, 97]),
    (32, 3, [200, 31, 97]),        # one wave's heads live, three idle
    (64, 2, [129, 300]),
    (96, 2, [64, 257]),
    (100, 2, [129, 40]),           # a partly live wave
    (256, 2, [150, 33]),           # two workgroups per sequence
    (128, 300, None),              # enough sequences to fill the GPU unsplit (no workspace)
])
def test_mla_head_counts(n_heads, batch, lens):
    say(f"case: MLA n_heads={n_heads} batch={batch} lens={lens}")
    ctx = 64 if lens is None else max(lens) + 5
    c = inputs.mla_case(11, batch=batch, ctx=ctx, n_heads=n_heads, seq_lens=lens)
    lat = c.latent.copy()
    for b, L in enumerate(c.seq_lens):
        lat[b, int(L):] = np.nan
    maxlen = int(max(c.seq_lens))
    o = host(pk.mla_decode_latent(dev(c.q_abs, "bf16"), dev(lat, "bf16"), i32(c.seq_lens),
                                  kv_lora_rank=512, max_seq_len=maxlen, attention_scale=c.scale))
    bsel = list(range(batch)) if batch <= 4 else [0, 1, batch // 2, batch - 1]
    ref = O.mla_decode_latent(c.q_abs, c.latent, c.seq_lens, 512, c.scale, batch_indices=bsel)
    check(o[bsel], ref, "bf16", f"MLA H={n_heads}")
    if lens is None:
        assert pk.mla_decode_workspace_size(batch, n_heads, 512, maxlen) == 0


def test_mla_zero_scale_is_the_mean_of_the_visible_values():
    lens = [1, 33, 700, 1500]
    say(f"case: MLA at attention_scale 0, lens={lens}")
    c = inputs.mla_case(9, batch=len(lens), ctx=1504, seq_lens=lens, n_heads=32)
    lat = c.latent.copy()
    for b, L in enumerate(lens):
        lat[b, L:] = np.nan
    o = pk.mla_decode_latent(dev(c.q_abs, "bf16"), dev(lat, "bf16"), i32(lens),
                             kv_lora_rank=512, max_seq_len=max(lens), attention_scale=0.0)
    ref = O.mla_decode_latent(c.q_abs, c.latent, lens, 512, 0.0)
    for b, L in enumerate(lens):
        mean = c.latent[b, :L, :512].astype(np.float64).mean(axis=0)
        assert np.allclose(ref[b], mean[None, :], atol=1e-12)
    check(host(o), ref, "bf16", "MLA scale 0")


def test_mla_bad_length_gives_nan():
    say("case: MLA with an out-of-range length")
    c = inputs.mla_case(5, batch=32, ctx=256)
    lens = c.seq_lens.copy()
    lens[4] = 300
    o = host(pk.mla_decode_latent(dev(c.q_abs, "bf16"), dev(c.latent, "bf16"), i32(lens),
                                  kv_lora_rank=512, max_seq_len=256, attention_scale=c.scale))
    assert np.all(np.isnan(o[4]))
    assert np.all(np.isfinite(np.delete(o, 4, axis=0)))


# ------------------------------------------------------------------ errors

def test_unknown_dtype_code_rejected_on_gpu():
    x = torch.zeros(16, device=DEV)
    st = pk.lib().attn_prefill(9, x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), 1, 1, 1,
                               16, 1, 1, 0, 1.0, None, 0, 0, 0, 1, None)
    assert st == 2
    with pytest.raises(TypeError):
        pk.attn_prefill(torch.zeros(1, 1, 1, 16, dtype=torch.float16, device=DEV),
                        torch.zeros(1, 1, 1, 16, dtype=torch.float16, device=DEV),
                        torch.zeros(1, 1, 1, 16, dtype=torch.float16, device=DEV),
                        seq_kv=1, position_offset=0, attention_scale=1.0)
