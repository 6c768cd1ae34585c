"""attn_decode_paged_noalloc: the allocation-free paged decode on the library's static scratch.

Called through the C-ABI binding and compared bitwise with attn_decode_paged (same
kernels, same partial layout, caller workspace) on two calls in a row, the second
with a smaller input, and with the float64 oracle on sampled sequences.
"""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_attention_causal_amd as pk
from oracle import oracle as O
from paged_kv_attention_causal_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
ESCRATCH = 5


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(DEV)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _both(c, sel):
    q, kp, vp = dev(c.q), dev(c.k_pool), dev(c.v_pool)
    bt, lens = i32(c.block_table), i32(c.seq_lens)
    maxlen = int(c.block_table.shape[1] * c.block_size)
    ref_call = pk.attn_decode_paged(q, kp, vp, bt, lens, max_seq_len=maxlen,
                                    attention_scale=c.scale)
    out = torch.full_like(q, float("nan"))
    pk.attn_decode_paged_noalloc(q, kp, vp, bt, lens, max_seq_len=maxlen,
                                 attention_scale=c.scale, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_call), "noalloc != attn_decode_paged (bitwise)"
    ref = O.decode_paged(c.q, c.k_pool, c.v_pool, c.block_table, c.block_size, c.seq_lens,
                         c.n_heads, c.n_kv_heads, c.scale, batch_indices=sel)
    err = np.abs(out.float().cpu().numpy().astype(np.float64)[sel] - ref).max()
    print(f"  max|err| vs oracle {err:.3e}", flush=True)
    assert err <= 2e-2


def test_noalloc_decode_twice_second_smaller():
    print("case: noalloc paged decode, 64 seqs L~U[512,8192] H=32 Hkv=8, then 5 seqs H=8 Hkv=2",
          flush=True)
    _both(inputs.paged_decode_case(0), [0, 17, 63])
    _both(inputs.paged_decode_case(8, batch=5, len_lo=100, len_hi=600, n_heads=8, n_kv_heads=2),
          [0, 1, 2, 3, 4])


def test_noalloc_decode_rejects_sizes_beyond_the_scratch():
    x = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    lens = torch.ones(1, dtype=torch.int32, device=DEV)
    bt = torch.zeros(1, dtype=torch.int32, device=DEV)
    p = ctypes.c_void_p
    # 4096 sequences x 32 heads x D=128 needs (2048 + 4096) x 32 x 130 x 4 B > 64 MiB;
    # rejected before anything is read or launched
    st = pk.lib().attn_decode_paged_noalloc(1, p(x.data_ptr()), p(x.data_ptr()), p(x.data_ptr()),
                                            p(x.data_ptr()), 4096, 32, 8, 128, p(bt.data_ptr()),
                                            512, 16, 1000, p(lens.data_ptr()), 8192, 0.088, None)
    assert st == ESCRATCH
    assert pk.status_string(ESCRATCH).startswith("sizes exceed")
