"""The hot-path calls captured in a HIP graph (torch.cuda.graph) and replayed.

Every entry point takes caller buffers and makes no allocation, memset or
host query after its first call on a device, so a serving loop can capture
it. Each case: one eager call to warm up, capture, then three replays with
the inputs changed in place between them (plus unrelated eager work), each
replay compared bitwise with an eager call on the same inputs. Covered:
paged decode (workspace and static scratch), the push followed by paged
decode, causal, chunked and ragged prefill, the MLA latent decode and its
two projections.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_causal_amd as pk
from paged_kv_attention_causal_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev(a, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype).to(DEV)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def say(*a):
    print(*a, flush=True)


def replay_and_compare(call, out, mutate, reps=3):
    """call() writes out; mutate(r) changes the inputs in place."""
    call()                                   # first call: per-device lookups happen here
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(reps):
        mutate(r)
        junk = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        out.fill_(float("nan"))
        call()                               # eager, same inputs
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(got, out), f"replay {r} != eager call"


def test_graph_paged_decode_with_workspace_and_noalloc():
    say("case: paged decode (caller workspace, and the static-scratch entry) in a graph")
    c = inputs.paged_decode_case(3, batch=16, len_lo=100, len_hi=3000, n_heads=32, n_kv_heads=8)
    q, kp, vp = dev(c.q), dev(c.k_pool), dev(c.v_pool)
    bt, lens = i32(c.block_table), i32(c.seq_lens)
    maxlen = int(c.block_table.shape[1] * c.block_size)
    ws = torch.empty(pk.attn_decode_workspace_size(16, 32, 8, 128, maxlen), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty_like(q)
    q2 = [dev(np.random.default_rng(40 + r).standard_normal(c.q.shape)) for r in range(3)]

    def call():
        pk.attn_decode_paged(q, kp, vp, bt, lens, max_seq_len=maxlen, attention_scale=c.scale,
                             out=out, workspace=ws)

    replay_and_compare(call, out, lambda r: q.copy_(q2[r]))
    out_na = torch.empty_like(q)

    def call_na():
        pk.attn_decode_paged_noalloc(q, kp, vp, bt, lens, max_seq_len=maxlen,
                                     attention_scale=c.scale, out=out_na)

    replay_and_compare(call_na, out_na, lambda r: q.copy_(q2[(r + 1) % 3]))


def test_graph_prefill_and_chunked_prefill():
    say("case: causal prefill and chunked paged prefill in graphs")
    c = inputs.prefill_case(5, batch=1, n_heads=8, n_kv_heads=2, seq_q=700)
    q, k, v = dev(c.q), dev(c.k), dev(c.v)
    out = torch.empty_like(q)
    q2 = [dev(np.random.default_rng(50 + r).standard_normal(c.q.shape) * 0.7) for r in range(3)]

    def call():
        pk.attn_prefill(q, k, v, seq_kv=c.seq_kv, position_offset=0, attention_scale=c.scale,
                        out=out)

    replay_and_compare(call, out, lambda r: q.copy_(q2[r]))
    cc = inputs.chunked_paged_prefill_case(2, batch=2, cached=600, seq_q=300)
    cq, ck, cv, cbt = dev(cc.q), dev(cc.k), dev(cc.v), i32(cc.block_table)
    cout = torch.empty_like(cq)
    k2 = [dev(np.random.default_rng(60 + r).standard_normal(cc.k.shape)) for r in range(3)]

    def call_c():
        pk.attn_prefill(cq, ck, cv, seq_kv=cc.seq_kv, position_offset=cc.position_offset,
                        attention_scale=cc.scale, block_table=cbt, out=cout)

    replay_and_compare(call_c, cout, lambda r: ck.copy_(k2[r]))


def test_graph_mla_latent_decode():
    say("case: MLA latent decode (split context, caller workspace) in a graph")
    lens = [2000, 700, 1500, 64]
    c = inputs.mla_case(7, batch=len(lens), ctx=2048, seq_lens=lens, n_heads=128)
    q, lat, ln = dev(c.q_abs), dev(c.latent), i32(lens)
    ws = torch.empty(pk.mla_decode_workspace_size(len(lens), 128, 512, 2048) + 16,
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((len(lens), 128, 512), dtype=torch.bfloat16, device=DEV)
    q2 = [dev(np.random.default_rng(70 + r).standard_normal(c.q_abs.shape)) for r in range(3)]

    def call():
        pk.mla_decode_latent(q, lat, ln, kv_lora_rank=512, max_seq_len=2048,
                             attention_scale=c.scale, out=out, workspace=ws)

    replay_and_compare(call, out, lambda r: q.copy_(q2[r]))


def test_graph_push_then_paged_decode():
    say("case: push of one K/V row per sequence, then paged decode, in one graph")
    c = inputs.append_case(0, held_hi=2047)
    kp, vp = dev(c.k_cache), dev(c.v_cache)
    bt, pos = i32(c.block_table), i32(c.held)
    kn, vn = dev(c.k_new), dev(c.v_new)
    lens = i32(c.held + 1)
    q = dev(inputs.paged_decode_case(5, batch=64, len_lo=1, len_hi=2, n_heads=32, n_kv_heads=8).q)
    maxlen = int(c.block_table.shape[1] * 16)
    ws = torch.empty(pk.attn_decode_workspace_size(64, 32, 8, 128, maxlen), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty_like(q)
    rng = np.random.default_rng(80)
    new_rows = [(dev(rng.standard_normal(c.k_new.shape)), dev(rng.standard_normal(c.v_new.shape)))
                for _ in range(3)]

    def call():
        pk.kv_append(kn, vn, kp, vp, pos, block_table=bt)
        pk.attn_decode_paged(q, kp, vp, bt, lens, max_seq_len=maxlen, attention_scale=1 / np.sqrt(128),
                             out=out, workspace=ws)

    def mutate(r):
        kn.copy_(new_rows[r][0])
        vn.copy_(new_rows[r][1])

    # The eager call after each replay writes the same rows again, so both read the same pool.
    replay_and_compare(call, out, mutate)


def test_graph_ragged_prefill_and_mla_projections():
    say("case: ragged paged prefill, and the MLA absorb and up-projection GEMMs, in graphs")
    r = inputs.varlen_prefill_case(6, batch=5, q_hi=300, cached_hi=700)
    rq, rk, rv, rbt = dev(r.q), dev(r.k), dev(r.v), i32(r.block_table)
    rcu, rkv = i32(r.cu_q), i32(r.seq_kv)
    rout = torch.empty_like(rq)
    q2 = [dev(np.random.default_rng(90 + i).standard_normal(r.q.shape)) for i in range(3)]

    def call():
        pk.attn_prefill_varlen(rq, rk, rv, rcu, rkv, max_seq_q=int(r.q_lens.max()),
                               attention_scale=r.scale, block_table=rbt, out=rout)

    replay_and_compare(call, rout, lambda i: rq.copy_(q2[i]))
    w = inputs.mla_proj_case(5, batch=8, n_heads=32)
    wq, wkb, wvb = dev(w.q), dev(w.k_b), dev(w.v_b)
    qa = torch.empty((8, 32, 576), dtype=torch.bfloat16, device=DEV)
    up = torch.empty((8, 32, wvb.shape[1]), dtype=torch.bfloat16, device=DEV)
    ol = dev(w.o_lat)
    q3 = [dev(np.random.default_rng(95 + i).standard_normal(w.q.shape)) for i in range(3)]

    def call_proj():
        pk.mla_absorb_q(wq, wkb, out=qa)
        pk.mla_up_proj(ol, wvb, out=up)

    replay_and_compare(call_proj, qa, lambda i: wq.copy_(q3[i]))
