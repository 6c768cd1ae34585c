"""GPU parity of the MLA pieces around the latent attention: the paged latent pool, the
absorb GEMM (q_nope . k_b[h]) and the value up-projection (v_b[h] . o_lat), each
against the float64 oracle, and the whole absorbed step against the oracle's
absorbed MLA."""
import numpy as np
import pytest
import torch

import paged_kv_attention_causal_amd as pk
from oracle import oracle as O
from paged_kv_attention_causal_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(DEV)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)


def check(got, ref, what, tol=2e-2):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) or 1.0
    say(f"  {what}: max|err|={err.max():.3e} max|err|/rms={err.max() / rms:.3e} rms={rms:.3e}")
    assert err.max() <= tol, f"{what}: {err.max():.3e}"


def to_pool(lat, lens, bs, rng, fill=np.nan):
    """Scatter contiguous latent rows [B, cap, W] into a shuffled pool of bs-row blocks."""
    B, W = lat.shape[0], lat.shape[2]
    need = [(int(L) + bs - 1) // bs for L in lens]
    nb = sum(need) + 5
    perm = rng.permutation(nb)
    bt = np.full((B, max(need)), -1, dtype=np.int32)
    pool = np.full((nb, bs, W), fill, dtype=np.float32)
    o = 0
    for b in range(B):
        for j in range(need[b]):
            bt[b, j] = perm[o]
            n = min(bs, int(lens[b]) - j * bs)
            pool[perm[o], :n] = lat[b, j * bs:j * bs + n]
            o += 1
    return pool, bt


@pytest.mark.parametrize("bs,lens,H", [(16, [4096] * 32, 128), (1, [1000, 37, 600], 128),
                                       (64, [1, 64, 65, 129, 2000], 32), (8, [300, 5000], 256),
                                       (16, [700, 33, 1500], 16)])
def test_mla_paged_latent_matches_contiguous_and_oracle(bs, lens, H):
    say(f"case: MLA paged latent bs={bs} lens={lens[:6]}{'...' if len(lens) > 6 else ''} H={H}")
    cap = max(lens)
    c = inputs.mla_case(3, batch=len(lens), ctx=cap, seq_lens=lens, n_heads=H)
    lat = c.latent.copy()
    for b, L in enumerate(lens):
        lat[b, L:] = np.nan
    pool, bt = to_pool(lat, lens, bs, np.random.default_rng(9))
    q = dev(c.q_abs)
    oc = pk.mla_decode_latent(q, dev(lat), i32(lens), kv_lora_rank=512, max_seq_len=cap,
                              attention_scale=c.scale)
    op = pk.mla_decode_latent_paged(q, dev(pool), i32(bt), i32(lens), kv_lora_rank=512,
                                    max_seq_len=cap, attention_scale=c.scale)
    assert torch.equal(op, oc), "paged latent != contiguous latent (bitwise)"
    sel = list(range(len(lens))) if len(lens) <= 5 else [0, 13, 31]
    ref = O.mla_decode_latent(c.q_abs, c.latent, lens, 512, c.scale, batch_indices=sel)
    check(host(op)[sel], ref, "paged latent decode")


def test_mla_paged_bad_block_gives_nan():
    say("case: MLA paged latent with an out-of-pool block id")
    lens = [700, 900, 50]
    c = inputs.mla_case(4, batch=3, ctx=900, seq_lens=lens, n_heads=128)
    pool, bt = to_pool(c.latent, lens, 16, np.random.default_rng(1))
    bt[1, 20] = pool.shape[0] + 2
    o = host(pk.mla_decode_latent_paged(dev(c.q_abs), dev(pool), i32(bt), i32(lens),
                                        kv_lora_rank=512, max_seq_len=900,
                                        attention_scale=c.scale))
    assert np.all(np.isnan(o[1]))
    ref = O.mla_decode_latent(c.q_abs, c.latent, lens, 512, c.scale, batch_indices=[0, 2])
    check(o[[0, 2]], ref, "clean sequences")


@pytest.mark.parametrize("B,H", [(32, 128), (5, 16), (33, 32)])
def test_mla_absorb_and_up_projection(B, H):
    say(f"case: MLA absorb and up-projection GEMMs B={B} H={H}")
    c = inputs.mla_proj_case(5, batch=B, n_heads=H)
    qa = pk.mla_absorb_q(dev(c.q), dev(c.k_b))
    check(host(qa), O.mla_absorb_q(c.q, c.k_b), "absorb")
    # the rope part is copied bit for bit
    assert np.array_equal(host(qa)[..., 512:], c.q[..., 128:].astype(np.float64))
    up = pk.mla_up_proj(dev(c.o_lat), dev(c.v_b))
    check(host(up), O.mla_up_proj(c.o_lat, c.v_b), "up-projection")


def test_mla_full_absorbed_step_against_naive_definition():
    """absorb -> paged latent attention -> up-projection on the GPU, against the oracle's
    absorbed MLA (itself pinned to the naive per-head form)."""
    B, H, L = 4, 128, 1500
    say(f"case: full absorbed MLA step B={B} H={H} ctx={L}")
    w = inputs.mla_proj_case(6, batch=B, n_heads=H)
    c = inputs.mla_case(7, batch=B, ctx=L, n_heads=H)
    lens = [L] * B
    pool, bt = to_pool(c.latent, lens, 16, np.random.default_rng(2))
    scale = 1 / np.sqrt(192)
    qa = pk.mla_absorb_q(dev(w.q), dev(w.k_b))
    o_lat = pk.mla_decode_latent_paged(qa, dev(pool), i32(bt), i32(lens), kv_lora_rank=512,
                                       max_seq_len=L, attention_scale=scale)
    out = host(pk.mla_up_proj(o_lat, dev(w.v_b)))
    for b in range(B):
        ref = O.mla_absorbed(w.q[b], c.latent[b, :, :512], c.latent[b, :, 512:],
                             np.transpose(w.k_b, (0, 2, 1)), w.v_b, scale)
        check(out[b], ref, f"sequence {b}")
