"""Pins for the float64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every check is a value the
pages print (tests/golden), a closed form, a library routine that computes
the same special case (torch's scaled_dot_product_attention on the CPU in
float64), an invariant, or the independent brute-force form.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kopitiam_attention_unit_values.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _vals(lst):
    return np.array([-np.inf if x == "-inf" else x for x in lst], dtype=np.float64)


# ---------------------------------------------------------------- page values

def test_golden_repeat_kv_heads_shares():
    g = _golden()["repeat_kv_heads_shares"]
    x = np.array(g["input"]).reshape(g["input_shape"])
    y = O.repeat_kv_heads(x, g["group_size"])
    assert list(y.shape) == g["expected_shape"]
    d = y.reshape(-1)
    assert d.tolist() == g["expected"]
    assert d[0] == d[1] and d[2] == d[3] and d[0] != d[2]


def test_golden_repeat_kv_heads_identity():
    g = _golden()["repeat_kv_heads_identity"]
    x = np.array(g["input"]).reshape(g["input_shape"])
    assert O.repeat_kv_heads(x, 1).reshape(-1).tolist() == g["expected"]


@pytest.mark.parametrize("key", ["mask_prefill_3x3", "mask_decode_offset"])
def test_golden_masks(key):
    g = _golden()[key]
    m = O.causal_mask(g["seq_q"], g["seq_kv"], g["position_offset"]).reshape(-1)
    exp = _vals(g["expected"])
    assert np.array_equal(m, exp)
    assert np.all(np.isneginf(m) == np.isneginf(exp))


def test_golden_mask_is_exact_neg_inf():
    g = _golden()["mask_exact_neg_inf"]
    m = O.causal_mask(g["seq_q"], g["seq_kv"], g["position_offset"]).reshape(-1)
    assert m[g["index"]] == -np.inf


def test_golden_masked_softmax_exact_zeros():
    g = _golden()["masked_softmax_zero_weight"]
    s = np.array(g["scores"]).reshape(1, 1, -1)
    p = O.masked_softmax(s, O.causal_mask(g["seq_q"], g["seq_kv"], g["position_offset"])).reshape(-1)
    assert abs(p[0] - 1.0) < g["atol_first"]
    assert p[1] == 0.0 and p[2] == 0.0


def test_golden_zero_kv_gives_zero_output():
    g = _golden()["zero_kv_zero_output"]
    x = (np.arange(g["seq"] * g["hidden"]) * 0.1).reshape(g["seq"], g["n_heads"], g["head_dim"])
    z = np.zeros((g["seq"], g["n_kv_heads"], g["head_dim"]))
    out = O.gqa_attention(x, z, z, g["n_heads"], g["n_kv_heads"], 0, 1 / math.sqrt(g["head_dim"]))
    assert out.shape == (g["seq"], g["n_heads"], g["head_dim"])
    assert np.all(out == 0.0)


# ------------------------------------------------------------ library routine

def _sdpa(q, k, v, n_heads, n_kv_heads, off, scale):
    """torch SDPA (float64, CPU) with enable_gqa and a boolean lower-triangular mask."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None].double()
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None].double()
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None].double()
    allowed = torch.ones(q.shape[0], k.shape[0], dtype=torch.bool).tril(diagonal=off)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=allowed, scale=scale, enable_gqa=(n_heads != n_kv_heads))
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("H,Hkv,D,Dv,sq,off,seed", [
    (4, 4, 8, 8, 9, 0, 0),       # plain MHA (group size 1)
    (6, 2, 16, 16, 17, 0, 1),    # GQA prefill
    (8, 2, 16, 16, 5, 11, 2),    # chunk after cached tokens
    (4, 1, 32, 24, 1, 40, 3),    # MQA decode, value width differs
    (28, 4, 128, 128, 33, 7, 4), # the large prefill's head layout
])
def test_oracle_matches_torch_sdpa(H, Hkv, D, Dv, sq, off, seed):
    rng = np.random.default_rng(seed)
    skv = off + sq
    q = rng.standard_normal((sq, H, D))
    k = rng.standard_normal((skv, Hkv, D))
    v = rng.standard_normal((skv, Hkv, Dv))
    scale = 0.3 + 0.1 * seed
    ref = _sdpa(q, k, v, H, Hkv, off, scale)
    got = O.gqa_attention(q, k, v, H, Hkv, off, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_sdpa_causal_flag_agrees_at_offset_zero():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((12, 4, 8))
    k = rng.standard_normal((12, 2, 8))
    v = rng.standard_normal((12, 2, 8))
    tq = torch.from_numpy(q.transpose(1, 0, 2).copy())[None]
    tk = torch.from_numpy(k.transpose(1, 0, 2).copy())[None]
    tv = torch.from_numpy(v.transpose(1, 0, 2).copy())[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.5,
                                                           enable_gqa=True)[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(O.gqa_attention(q, k, v, 4, 2, 0, 0.5), ref, rtol=0, atol=1e-12)


# -------------------------------------------------------------- closed forms

def test_two_key_closed_form():
    # scores (0, ln 3) give weights (1/4, 3/4); the query at position 1 sees both keys.
    q = np.array([[[1.0]]])
    k = np.array([[[0.0]], [[math.log(3.0)]]])
    v = np.array([[[4.0, -8.0]], [[8.0, 4.0]]])
    got = O.gqa_attention(q, k, v, 1, 1, 1, 1.0)[0, 0]
    np.testing.assert_allclose(got, [7.0, 1.0], rtol=0, atol=1e-14)
    # The same query at position 0 may see key 0 only: output is v[0].
    got0 = O.gqa_attention(q, k, v, 1, 1, 0, 1.0)[0, 0]
    assert np.array_equal(got0, v[0, 0])


def test_zero_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(11)
    sq, off, H, Hkv, D = 6, 3, 4, 2, 5
    q = rng.standard_normal((sq, H, D))
    k = np.zeros((off + sq, Hkv, D))
    v = rng.standard_normal((off + sq, Hkv, D))
    out = O.gqa_attention(q, k, v, H, Hkv, off, 0.7)
    for i in range(sq):
        for h in range(H):
            np.testing.assert_allclose(out[i, h], v[:off + i + 1, h // (H // Hkv)].mean(axis=0),
                                       rtol=0, atol=1e-14)


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((7, 6, 4))
    k = rng.standard_normal((7, 3, 4))
    v = np.full((7, 3, 4), -2.5)
    assert np.allclose(O.gqa_attention(q, k, v, 6, 3, 0, 1.3), -2.5, rtol=0, atol=1e-14)
    assert np.all(O.gqa_attention(q, k, np.zeros_like(v), 6, 3, 0, 1.3) == 0.0)


def test_first_row_is_first_value_of_its_kv_head():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((5, 8, 3))
    k = rng.standard_normal((5, 2, 3))
    v = rng.standard_normal((5, 2, 3))
    out = O.gqa_attention(q, k, v, 8, 2, 0, 2.0)
    for h in range(8):
        assert np.array_equal(out[0, h], v[0, h // 4])


def test_hard_attention_limit_picks_the_best_key():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 2, 6))
    k = rng.standard_normal((9, 1, 6))
    v = rng.standard_normal((9, 1, 6))
    out = O.gqa_attention(q, k, v, 2, 1, 8, 1e4)
    for h in range(2):
        j = int(np.argmax(k[:, 0] @ q[0, h]))
        np.testing.assert_allclose(out[0, h], v[j, 0], rtol=0, atol=1e-9)


# ------------------------------------------------------------------ invariants

def test_group_members_share_kv_and_only_their_group_moves():
    rng = np.random.default_rng(15)
    H, Hkv, G, D = 6, 3, 2, 4
    qrow = rng.standard_normal((4, 1, D))
    q = np.repeat(qrow, H, axis=1)          # identical query in every head
    k = rng.standard_normal((4, Hkv, D))
    v = rng.standard_normal((4, Hkv, D))
    base = O.gqa_attention(q, k, v, H, Hkv, 0, 0.5)
    for g in range(Hkv):
        for h in range(g * G, (g + 1) * G):
            assert np.array_equal(base[:, h], base[:, g * G])
    k2, v2 = k.copy(), v.copy()
    k2[:, 1] += 1.0
    v2[:, 1] -= 0.5
    moved = O.gqa_attention(q, k2, v2, H, Hkv, 0, 0.5)
    for h in range(H):
        same = np.array_equal(moved[:, h], base[:, h])
        assert same == (h // G != 1), h


def test_outputs_are_convex_combinations_of_visible_values():
    rng = np.random.default_rng(16)
    sq, off, H, Hkv, D = 5, 4, 4, 4, 6
    q = rng.standard_normal((sq, H, D)) * 3
    k = rng.standard_normal((off + sq, Hkv, D))
    v = rng.standard_normal((off + sq, Hkv, D))
    out = O.gqa_attention(q, k, v, H, Hkv, off, 1.0)
    for i in range(sq):
        vis = v[:off + i + 1]
        assert np.all(out[i] <= vis.max(axis=0) + 1e-12)
        assert np.all(out[i] >= vis.min(axis=0) - 1e-12)


def test_decode_step_equals_prefill_row():
    rng = np.random.default_rng(17)
    T, H, Hkv, D = 20, 4, 2, 8
    q = rng.standard_normal((1, T, H, D))
    k = rng.standard_normal((1, T, Hkv, D))
    v = rng.standard_normal((1, T, Hkv, D))
    full = O.prefill(q, k, v, H, Hkv, T, 0, 0.4)
    for L in range(1, T + 1):
        dec = O.decode_contig(q[:, L - 1], k, v, [L], H, Hkv, 0.4)
        np.testing.assert_allclose(dec[0], full[0, L - 1], rtol=0, atol=1e-13)


def test_paged_equals_contiguous_and_is_block_permutation_invariant():
    from paged_kv_attention_causal_amd import inputs
    case = inputs.paged_decode_case(3, dtype="f32", batch=5, len_lo=1, len_hi=70, n_heads=4,
                                    n_kv_heads=2, head_dim=8, block_size=16)
    kc, vc = case.contig()
    a = O.decode_paged(case.q, case.k_pool, case.v_pool, case.block_table, 16, case.seq_lens, 4, 2,
                       case.scale)
    b = O.decode_contig(case.q, kc, vc, case.seq_lens, 4, 2, case.scale)
    assert np.array_equal(a, b)
    # Permute the pool's blocks and rename the table entries to match.
    rng = np.random.default_rng(99)
    perm = rng.permutation(case.k_pool.shape[0])
    inv = np.argsort(perm)
    kp2, vp2 = case.k_pool[perm], case.v_pool[perm]
    bt2 = np.where(case.block_table >= 0, inv[np.maximum(case.block_table, 0)], -1)
    c = O.decode_paged(case.q, kp2, vp2, bt2, 16, case.seq_lens, 4, 2, case.scale)
    assert np.array_equal(a, c)


def test_paged_prefill_equals_contiguous_prefill():
    from paged_kv_attention_causal_amd import inputs
    case = inputs.chunked_paged_prefill_case(5, dtype="f32", batch=2, cached=21, seq_q=11, n_heads=4,
                                             n_kv_heads=2, head_dim=8, block_size=4, scale=0.3)
    paged = O.prefill(case.q, case.k, case.v, 4, 2, case.seq_kv, case.position_offset, case.scale,
                      block_table=case.block_table, block_size=case.block_size)
    kc = np.stack([O.gather_paged(case.k, case.block_table[b], 4, case.seq_kv) for b in range(2)])
    vc = np.stack([O.gather_paged(case.v, case.block_table[b], 4, case.seq_kv) for b in range(2)])
    contig = O.prefill(case.q, kc, vc, 4, 2, case.seq_kv, case.position_offset, case.scale)
    assert np.array_equal(paged, contig)
    rows = O.prefill(case.q, kc, vc, 4, 2, case.seq_kv, case.position_offset, case.scale,
                     rows=[0, 5, 10])
    np.testing.assert_allclose(rows, contig[:, [0, 5, 10]], rtol=0, atol=1e-13)


# --------------------------------------------------------------------- brute

@pytest.mark.parametrize("seed", range(12))
def test_brute_force_agrees(seed):
    rng = np.random.default_rng(100 + seed)
    H = int(rng.choice([1, 2, 4, 6]))
    divs = [d for d in range(1, H + 1) if H % d == 0]
    Hkv = int(rng.choice(divs))
    D = int(rng.choice([1, 3, 8]))
    sq = int(rng.integers(1, 6))
    off = int(rng.integers(0, 5))
    skv = off + sq + int(rng.integers(-min(off, 2), 3))   # also seq_kv != off + seq_q
    skv = max(skv, 1)
    q = rng.standard_normal((sq, H, D))
    k = rng.standard_normal((skv, Hkv, D))
    v = rng.standard_normal((skv, Hkv, D))
    scale = float(rng.uniform(0.1, 2.0))
    got = O.gqa_attention(q, k, v, H, Hkv, off, scale)
    ref = np.array(brute.gqa_attention(q.tolist(), k.tolist(), v.tolist(), H, Hkv, off, scale))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_oracle_rejects_bad_head_counts():
    q = np.zeros((1, 3, 2))
    kv = np.zeros((1, 2, 2))
    with pytest.raises(ValueError):
        O.gqa_attention(q, kv, kv, 3, 2, 0, 1.0)
    with pytest.raises(ValueError):
        O.gqa_attention(q, np.zeros((1, 0, 2)), np.zeros((1, 0, 2)), 3, 0, 0, 1.0)


# ----------------------------------------------------------------------- MLA

def test_mla_absorbed_equals_naive():
    rng = np.random.default_rng(21)
    H, R, P, nope, vdim, L = 4, 16, 8, 8, 8, 13
    q = rng.standard_normal((H, nope + P))
    c = rng.standard_normal((L, R))
    k_rot = rng.standard_normal((L, P))
    w_uk = rng.standard_normal((H, nope, R)) * 0.3
    w_uv = rng.standard_normal((H, vdim, R)) * 0.3
    scale = 1.0 / math.sqrt(nope + P)
    naive = O.mla_naive(q, c, k_rot, w_uk, w_uv, scale)
    absorbed = O.mla_absorbed(q, c, k_rot, w_uk, w_uv, scale)
    np.testing.assert_allclose(absorbed, naive, rtol=0, atol=1e-12)


def test_mla_latent_matches_torch_sdpa_mqa():
    rng = np.random.default_rng(22)
    B, H, R, P, cap = 2, 8, 24, 8, 19
    q = rng.standard_normal((B, H, R + P))
    lat = rng.standard_normal((B, cap, R + P))
    lens = [19, 7]
    got = O.mla_decode_latent(q, lat, lens, R, 0.2)
    for b, L in enumerate(lens):
        tq = torch.from_numpy(q[b])[None, :, None, :]               # [1,H,1,R+P]
        tk = torch.from_numpy(lat[b, :L])[None, None]               # [1,1,L,R+P]
        tv = torch.from_numpy(lat[b, :L, :R].copy())[None, None]    # [1,1,L,R]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.2,
                                                               enable_gqa=True)[0, :, 0].numpy()
        np.testing.assert_allclose(got[b], ref, rtol=0, atol=1e-12)


def test_mla_value_is_the_leading_latent_slice():
    # With a zero query every position weighs the same: o_lat is the mean of latent[:, :R].
    rng = np.random.default_rng(23)
    lat = rng.standard_normal((1, 6, 12))
    out = O.mla_decode_latent(np.zeros((1, 3, 12)), lat, [6], 9, 0.5)
    np.testing.assert_allclose(out[0], np.broadcast_to(lat[0, :, :9].mean(0), (3, 9)), atol=1e-14)


# ---------------------------------------------------------------- cache append and RoPE

ROPE_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rope_append_values.json")


def _rope_golden():
    with open(ROPE_GOLDEN) as f:
        return json.load(f)


def test_golden_rope_unit_vectors():
    g = _rope_golden()["rope"]
    for c in g["cases"]:
        x = np.zeros(g["width"])
        x[c["unit"]] = 1.0
        y = O.rope_interleaved(x, c["position"], g["theta"])
        np.testing.assert_allclose(y[c["expect_at"]], c["expect"], rtol=0, atol=1e-15)
        # only the unit's own pair moves (interleaved pairs, not split halves)
        rest = np.delete(y, c["expect_at"])
        assert np.all(rest == 0.0)


def test_rope_identity_at_zero_norm_composition_and_broadcast():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64))
    assert np.array_equal(O.rope_interleaved(x, np.zeros(5), 1e4), x)
    pos = np.arange(5) * 37.0
    y = O.rope_interleaved(x, pos, 1e4)
    np.testing.assert_allclose(np.hypot(y[:, 0::2], y[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]),
                               rtol=1e-13)
    z = O.rope_interleaved(O.rope_interleaved(x, pos, 1e4), pos + 3.0, 1e4)
    np.testing.assert_allclose(z, O.rope_interleaved(x, 2 * pos + 3.0, 1e4), atol=1e-11)
    # rotating the shared vector once, then copying it to every head, equals
    # rotating every head's copy (the angle depends on the position only)
    heads = np.broadcast_to(x[:, None, :], (5, 3, 64))
    np.testing.assert_array_equal(O.rope_interleaved(heads, pos[:, None], 1e4),
                                  np.broadcast_to(y[:, None, :], (5, 3, 64)))


def test_golden_append_paged_and_contiguous():
    g = _rope_golden()["append_paged"]
    pool = np.zeros((g["num_blocks"], g["block_size"], 1))
    rows = np.array(g["new_rows"], dtype=np.float64)[:, :, None]
    out = O.append_rows(pool, rows, g["positions"], np.array(g["block_table"]), g["block_size"])
    expect = np.zeros_like(pool)
    for e in g["expect"]:
        expect[e["block"], e["row"], 0] = e["value"]
    assert np.array_equal(out, expect)
    g = _rope_golden()["append_contiguous"]
    cache = np.zeros((2, g["capacity"], 1))
    out = O.append_rows(cache, np.array(g["new_rows"])[:, :, None], g["positions"])
    expect = np.zeros_like(cache)
    for e in g["expect"]:
        expect[e["seq"], e["token"], 0] = e["value"]
    assert np.array_equal(out, expect)


def test_append_then_gather_is_old_rows_then_new_rows():
    rng = np.random.default_rng(4)
    B, bs, Hkv, D = 3, 4, 2, 5
    held = np.array([0, 5, 8])
    n_new = 3
    need = (held + n_new + bs - 1) // bs
    nb = int(need.sum()) + 2
    perm = rng.permutation(nb)
    bt = np.full((B, int(need.max())), -1)
    o = 0
    for b in range(B):
        bt[b, :need[b]] = perm[o:o + need[b]]
        o += need[b]
    pool = rng.standard_normal((nb, bs, Hkv, D))
    new = rng.standard_normal((B, n_new, Hkv, D))
    out = O.append_rows(pool, new, held, bt, bs)
    written = np.zeros((nb, bs), dtype=bool)
    for b in range(B):
        before = O.gather_paged(pool, bt[b], bs, int(held[b]))
        after = O.gather_paged(out, bt[b], bs, int(held[b]) + n_new)
        assert np.array_equal(after[:held[b]], before)
        assert np.array_equal(after[held[b]:], new[b])
        for t in range(held[b], held[b] + n_new):
            written[bt[b][t // bs], t % bs] = True
    # every other pool row is untouched
    assert np.array_equal(out[~written], pool[~written])
    # the contiguous form of the same push gathers to the same rows
    cap = int(held.max()) + n_new
    cont = np.zeros((B, cap, Hkv, D))
    for b in range(B):
        cont[b, :held[b]] = O.gather_paged(pool, bt[b], bs, int(held[b]))
    cont = O.append_rows(cont, new, held)
    for b in range(B):
        L = int(held[b]) + n_new
        assert np.array_equal(cont[b, :L], O.gather_paged(out, bt[b], bs, L))


def test_mla_append_latent_row_layout_and_attention():
    rng = np.random.default_rng(6)
    R, P, H, nope, vdim, L = 16, 8, 4, 8, 8, 6
    theta = 1e4
    c_hist = rng.standard_normal((L - 1, R))
    kr_hist = rng.standard_normal((L - 1, P))
    pos_hist = np.arange(L - 1)
    latent = np.zeros((1, L + 2, R + P))
    latent[0, :L - 1] = np.concatenate([c_hist, O.rope_interleaved(kr_hist, pos_hist, theta)], 1)
    c_new = rng.standard_normal((1, R))
    kr_new = rng.standard_normal((1, P))
    out = O.mla_append_latent(latent, c_new, kr_new, [L - 1], theta)
    assert np.array_equal(out[0, L - 1, :R], c_new[0])
    np.testing.assert_array_equal(out[0, L - 1, R:], O.rope_interleaved(kr_new[0], L - 1, theta))
    assert np.array_equal(out[0, :L - 1], latent[0, :L - 1]) and np.all(out[0, L:] == 0)
    # theta <= 0: the rope-free configuration stores k_rot as given
    raw = O.mla_append_latent(latent, c_new, kr_new, [L - 1], 0.0)
    assert np.array_equal(raw[0, L - 1, R:], kr_new[0])
    # attention over the appended latent (absorbed) equals the naive form in which
    # every head's key carries its own rotated copy of k_rot
    q = rng.standard_normal((H, nope + P))
    w_uk = rng.standard_normal((H, nope, R))
    w_uv = rng.standard_normal((H, vdim, R))
    c_all = out[0, :L, :R]
    kr_all = out[0, :L, R:]
    scale = 1 / math.sqrt(nope + P)
    absorbed = O.mla_absorbed(q, c_all, kr_all, w_uk, w_uv, scale)
    kr_raw = np.concatenate([kr_hist, kr_new], 0)
    per_head = O.rope_interleaved(np.broadcast_to(kr_raw[:, None, :], (L, H, P)),
                                  np.arange(L)[:, None], theta)
    keys = np.concatenate([np.einsum("hnr,lr->lhn", w_uk, c_all), per_head], axis=2)
    vals = np.einsum("hvr,lr->lhv", w_uv, c_all)
    naive = O.gqa_attention(q[None], keys, vals, H, H, L - 1, scale)[0]
    np.testing.assert_allclose(absorbed, naive, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- ragged prefill

def test_prefill_varlen_reduces_to_batched_and_to_brute_force():
    rng = np.random.default_rng(8)
    H, Hkv, D = 4, 2, 3
    # equal chunks and histories: the batched prefill
    B, n, held = 3, 4, 5
    q = rng.standard_normal((B, n, H, D))
    k = rng.standard_normal((B, held + n, Hkv, D))
    v = rng.standard_normal((B, held + n, Hkv, D))
    cu = np.arange(B + 1) * n
    got = O.prefill_varlen(q.reshape(B * n, H, D), k, v, cu, [held + n] * B, H, Hkv, 0.7)
    ref = O.prefill(q, k, v, H, Hkv, held + n, held, 0.7)
    np.testing.assert_allclose(got, ref.reshape(B * n, H, D), rtol=0, atol=1e-14)
    # ragged: every row against the scalar brute force at its own position
    lens, hist = [0, 3, 1, 5], [4, 0, 7, 2]
    cu = np.concatenate([[0], np.cumsum(lens)])
    skv = [a + b for a, b in zip(lens, hist)]
    q = rng.standard_normal((cu[-1], H, D))
    k = rng.standard_normal((4, max(skv), Hkv, D))
    v = rng.standard_normal((4, max(skv), Hkv, D))
    got = O.prefill_varlen(q, k, v, cu, skv, H, Hkv, 0.9)
    for b in range(4):
        for i in range(lens[b]):
            r = cu[b] + i
            exp = brute.gqa_attention(q[r:r + 1].tolist(), k[b, :skv[b]].tolist(),
                                  v[b, :skv[b]].tolist(), H, Hkv, hist[b] + i, 0.9)
            np.testing.assert_allclose(got[r], np.array(exp)[0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- attention arms

def test_arms_off_is_the_plain_definition():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((5, 4, 8))
    k = rng.standard_normal((9, 2, 8))
    v = rng.standard_normal((9, 2, 6))          # V narrower than K
    a = O.gqa_attention_arms(q, k, v, 4, 2, 4, 0.4)
    b = O.gqa_attention(q, k, v, 4, 2, 4, 0.4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
    # a window wider than every distance, zero slopes, a sink at -inf: still plain
    c = O.gqa_attention_arms(q, k, v, 4, 2, 4, 0.4, window=100, alibi=np.zeros(4),
                             sinks=np.full(4, -np.inf))
    np.testing.assert_allclose(c, b, rtol=0, atol=1e-14)


def test_arms_window_is_attention_over_the_last_keys():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 2, 4))
    k = rng.standard_normal((10, 1, 4))
    v = rng.standard_normal((10, 1, 4))
    for w in (1, 3, 7):
        got = O.gqa_attention_arms(q, k, v, 2, 1, 9, 0.5, window=w)
        # the plain attention over keys 10-w .. 9, the query being the last of them
        ref = O.gqa_attention(q, k[10 - w:], v[10 - w:], 2, 1, w - 1, 0.5)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)
    # window 1: the query sees its own key only
    np.testing.assert_array_equal(O.gqa_attention_arms(q, k, v, 2, 1, 9, 0.5, window=1)[0],
                                  np.repeat(v[9], 2, axis=0))


def test_arms_closed_forms_alibi_sinks_softcap():
    n = 6
    v = np.eye(n)[:, None, :]                   # one-hot values: the output is the weights
    k = np.zeros((n, 1, 3))
    q = np.zeros((1, 1, 3))
    # zero scores + ALiBi slope m: weights proportional to exp(-m (p - j)), geometric
    m = 0.7
    got = O.gqa_attention_arms(q, k, v, 1, 1, n - 1, 1.0, alibi=[m])[0, 0]
    r = [math.exp(-m * (n - 1 - j)) for j in range(n)]
    np.testing.assert_allclose(got, np.array(r) / sum(r), rtol=1e-14)
    # zero scores + a sink s: every key weighs 1 / (n + e^s)
    s = 1.3
    got = O.gqa_attention_arms(q, k, v, 1, 1, n - 1, 1.0, sinks=[s])[0, 0]
    np.testing.assert_allclose(got, np.full(n, 1 / (n + math.exp(s))), rtol=1e-14)
    # two keys with q.k = 0 and 2, scale 1, softcap 1: logits tanh(0) = 0 and tanh(2)
    q2 = np.array([[[1.0, 0.0]]])
    k2 = np.array([[[0.0, 0.0]], [[2.0, 0.0]]])
    v2 = np.eye(2)[:, None, :]
    got = O.gqa_attention_arms(q2, k2, v2, 1, 1, 1, 1.0, softcap=1.0)[0, 0]
    e = math.exp(math.tanh(2.0))
    np.testing.assert_allclose(got, [1 / (1 + e), e / (1 + e)], rtol=1e-14)
    # a huge cap is the plain softmax
    big = O.gqa_attention_arms(q2, k2, v2, 1, 1, 1, 1.0, softcap=1e7)[0, 0]
    np.testing.assert_allclose(big, [1 / (1 + math.e ** 2), math.e ** 2 / (1 + math.e ** 2)],
                               rtol=1e-9)


def test_arms_match_the_scalar_brute_force():
    rng = np.random.default_rng(13)
    for trial in range(8):
        H, Hkv = [(2, 1), (4, 2), (3, 3), (6, 2)][trial % 4]
        D, Dv = 1 + trial % 4, 1 + (trial * 3) % 5
        sq, off = 1 + trial % 3, trial % 5
        skv = off + sq + (trial % 2)
        q = rng.standard_normal((sq, H, D))
        k = rng.standard_normal((skv, Hkv, D))
        v = rng.standard_normal((skv, Hkv, Dv))
        kw = dict(window=[0, 2, 3, 1][trial % 4], softcap=[0.0, 0.8, 3.0, 0.0][(trial + 1) % 4],
                  alibi=rng.uniform(0, 1, H) if trial % 2 else None,
                  sinks=rng.standard_normal(H) if trial % 3 else None)
        got = O.gqa_attention_arms(q, k, v, H, Hkv, off, 0.6, **kw)
        ref = brute.gqa_attention_arms(q.tolist(), k.tolist(), v.tolist(), H, Hkv, off, 0.6, **kw)
        np.testing.assert_allclose(got, np.array(ref), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- MLA projections

def test_mla_projection_closed_forms():
    rng = np.random.default_rng(14)
    B, H, nope, P, R, vd = 2, 3, 4, 2, 5, 3
    q = rng.standard_normal((B, H, nope + P))
    # k_b[h] = e_{r, n}: q_abs[.., r] picks q_nope[n]; the rope part is copied
    k_b = np.zeros((H, R, nope))
    for h in range(H):
        k_b[h, (h + 1) % R, h % nope] = 2.0
    qa = O.mla_absorb_q(q, k_b)
    assert qa.shape == (B, H, R + P)
    for h in range(H):
        expect = np.zeros((B, R))
        expect[:, (h + 1) % R] = 2.0 * q[:, h, h % nope]
        np.testing.assert_array_equal(qa[:, h, :R], expect)
    np.testing.assert_array_equal(qa[..., R:], q[..., nope:])
    # up-projection by a per-head diagonal scales each latent entry
    o = rng.standard_normal((B, H, R))
    v_b = np.zeros((H, vd, R))
    for h in range(H):
        for i in range(vd):
            v_b[h, i, i] = h + 1.0
    np.testing.assert_array_equal(O.mla_up_proj(o, v_b), o[..., :vd] * (np.arange(H) + 1.0)[:, None])
