"""GPU parity of the decode arms (window, softcap, ALiBi, sinks, V narrower than K).

attn_decode_contig_ext / attn_decode_paged_ext against the float64 oracle's
decode_arms on the same seeded inputs; contiguous and paged must agree bitwise.
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


def dev(a, dtype="bf16"):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).to(DEV)


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)


def check(got, ref, dtype, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) or 1.0
    say(f"  {what}: max|err|={err.max():.3e} max|err|/rms={err.max() / rms:.3e}")
    assert err.max() <= TOL[dtype], f"{what}: {err.max():.3e}"


ARMS = {
    "off": {},
    "window": dict(window=100),
    "softcap": dict(softcap=1.5),
    "alibi": dict(alibi=True),
    "sinks": dict(sinks=True),
    "all": dict(window=300, softcap=2.0, alibi=True, sinks=True),
}


def _run(c, dtype, arms, H, kc=None, vc=None):
    kw = dict(window=arms.get("window", 0), softcap=arms.get("softcap", 0.0))
    alibi = inputs.alibi_slopes(H) if arms.get("alibi") else None
    sinks = inputs.sink_logits(3, H) if arms.get("sinks") else None
    maxlen = int(c.block_table.shape[1] * c.block_size)
    op = pk.attn_decode_paged_ext(dev(c.q, dtype), dev(c.k_pool, dtype), dev(c.v_pool, dtype),
                                  i32(c.block_table), i32(c.seq_lens), max_seq_len=maxlen,
                                  attention_scale=c.scale,
                                  alibi=None if alibi is None else f32(alibi),
                                  sinks=None if sinks is None else f32(sinks), **kw)
    oc = None
    if kc is not None:
        oc = pk.attn_decode_contig_ext(dev(c.q, dtype), dev(kc, dtype), dev(vc, dtype),
                                       i32(c.seq_lens), max_seq_len=maxlen,
                                       attention_scale=c.scale,
                                       alibi=None if alibi is None else f32(alibi),
                                       sinks=None if sinks is None else f32(sinks), **kw)
    ref_kw = dict(kw, alibi=alibi, sinks=sinks)
    return op, oc, ref_kw


@pytest.mark.parametrize("arm", list(ARMS))
@pytest.mark.parametrize("dtype,D,Dv,H,Hkv", [("bf16", 128, 128, 32, 8), ("bf16", 192, 128, 16, 2),
                                              ("f32", 16, 16, 6, 3), ("bf16", 192, 128, 8, 8)])
def test_decode_arms(arm, dtype, D, Dv, H, Hkv):
    lens = [1, 2, 99, 100, 101, 301, 700, 1500]
    say(f"case: decode arms={arm} {dtype} K={D} V={Dv} H={H} Hkv={Hkv} lens={lens}")
    c = inputs.paged_decode_case(41, dtype=dtype, batch=len(lens), n_heads=H, n_kv_heads=Hkv,
                                 head_dim=D, v_head_dim=Dv, block_size=16, seq_lens=lens,
                                 len_hi=1536, scale=0.3 if dtype == "f32" else None)
    kc, vc = c.contig(capacity=1536, fill=np.nan)
    op, oc, ref_kw = _run(c, dtype, ARMS[arm], H, kc, vc)
    assert torch.equal(op, oc), "contiguous != paged (bitwise)"
    ref = O.decode_arms(c.q, kc, vc, c.seq_lens, H, Hkv, c.scale, **ref_kw)
    check(host(op), ref, dtype, f"arms {arm}")


def test_decode_arms_full_size_all_arms():
    say("case: paged decode bf16 64 seqs L~U[512,8192] with window 4096, softcap 30, ALiBi, sinks")
    c = inputs.paged_decode_case(0)
    arms = dict(window=4096, softcap=30.0, alibi=True, sinks=True)
    op, _, ref_kw = _run(c, "bf16", arms, 32)
    op2, _, _ = _run(c, "bf16", arms, 32)
    assert torch.equal(op, op2), "not deterministic"
    sel = [0, 5, 33, 63]
    ref = O.decode_arms(c.q, c.k_pool, c.v_pool, c.seq_lens, 32, 8, c.scale, c.block_table, 16,
                        batch_indices=sel, **ref_kw)
    check(host(op)[sel], ref, "bf16", "full size, all arms")


def test_decode_arms_bad_length_gives_nan():
    c = inputs.paged_decode_case(8, batch=4, len_lo=100, len_hi=600, n_heads=8, n_kv_heads=2)
    lens = c.seq_lens.copy()
    lens[2] = 0
    o = host(pk.attn_decode_paged_ext(dev(c.q), dev(c.k_pool), dev(c.v_pool), i32(c.block_table),
                                      i32(lens), max_seq_len=600, attention_scale=c.scale,
                                      window=50, sinks=f32(inputs.sink_logits(1, 8))))
    assert np.all(np.isnan(o[2])) and np.all(np.isfinite(np.delete(o, 2, axis=0)))
