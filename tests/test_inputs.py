"""The seeded input generators: bf16 rounding, block tables, append cases, config shapes."""
import numpy as np
import pytest
import torch

from paged_kv_attention_causal_amd import inputs


def test_bf16_round_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(10_000) * 1e30).astype(np.float32),
        (rng.standard_normal(10_000) * 1e-38).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 3.4e38, -3.4e38, np.inf, -np.inf], dtype=np.float32),
        # exact ties: low 16 bits == 0x8000 with even and odd kept halves
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF, 0x3F807FFF],
                 dtype=np.uint32).view(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = inputs.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    nan = inputs.bf16_round(np.array([np.nan], dtype=np.float32))
    assert np.isnan(nan[0])


def test_block_tables_are_a_non_overlapping_draw_with_slack():
    rng = np.random.default_rng(1)
    lens = np.array([1, 16, 17, 100, 512])
    nb, bt = inputs.draw_block_tables(rng, lens, 16, 0.10)
    need = (lens + 15) // 16
    assert nb == int(np.ceil(1.1 * need.sum()))
    used = []
    for b, n in enumerate(need):
        assert np.all(bt[b, :n] >= 0) and np.all(bt[b, :n] < nb)
        assert np.all(bt[b, n:] == -1)
        used.extend(bt[b, :n].tolist())
    assert len(used) == len(set(used))


def test_paged_decode_full_size_recipe_seed0():
    # Only the cheap parts of the full paged-decode draw: lengths and table sizes.
    rng = np.random.default_rng(0)
    lens = rng.integers(512, 8193, size=64)
    assert lens.min() >= 512 and lens.max() <= 8192
    nb, bt = inputs.draw_block_tables(rng, lens, 16, 0.10, 512)
    assert bt.shape == (64, 512)
    assert nb == int(np.ceil(1.1 * ((lens + 15) // 16).sum()))


def test_append_cases_hold_history_and_nan_beyond():
    c = inputs.append_case(3, batch=4, n_new=3, held_lo=0, held_hi=40, n_kv_heads=2, head_dim=8,
                           block_size=4)
    for b in range(4):
        h = int(c.held[b])
        for t in range(h + 3):
            row = c.k_cache[c.block_table[b, t // 4], t % 4]
            assert np.all(np.isfinite(row)) == (t < h)
    m = inputs.mla_append_case(3, batch=3, held=[0, 5, 9], kv_lora_rank=16, qk_rope_head_dim=8)
    assert m.latent.shape == (3, 10, 24) and m.c_new.shape == (3, 16) and m.k_rot_new.shape == (3, 8)
    assert np.all(np.isnan(m.latent[0])) and np.all(np.isfinite(m.latent[2, :9]))


def test_small_case_shapes_and_storage_rounding():
    c = inputs.prefill_case(0, batch=2, n_heads=4, n_kv_heads=2, head_dim=16, seq_q=10,
                            position_offset=3)
    assert c.q.shape == (2, 10, 4, 16) and c.k.shape == (2, 13, 2, 16) and c.seq_kv == 13
    assert np.all((c.q.view(np.uint32) & 0xFFFF) == 0)
    d = inputs.paged_decode_case(0, dtype="f32", batch=3, len_lo=5, len_hi=40, n_heads=4,
                                 n_kv_heads=2, head_dim=8, block_size=16)
    kc, vc = d.contig()
    assert kc.shape == (3, int(d.seq_lens.max()), 2, 8)
    m = inputs.mla_case(0, batch=2, ctx=8, n_heads=4, kv_lora_rank=16, qk_rope_head_dim=8)
    assert m.latent.shape == (2, 8, 24) and m.q_abs.shape == (2, 4, 24)
    assert abs(m.scale - 1 / np.sqrt(192)) < 1e-15
    q, k, v, s = inputs.tiny_f32(0)
    assert q.shape == (1, 72, 4, 16) and k.shape == (1, 72, 2, 16) and s == 0.25


def test_generators_are_deterministic():
    a = inputs.paged_decode_case(4, batch=3, len_lo=5, len_hi=40, n_heads=4, n_kv_heads=2,
                                 head_dim=8, block_size=4)
    b = inputs.paged_decode_case(4, batch=3, len_lo=5, len_hi=40, n_heads=4, n_kv_heads=2,
                                 head_dim=8, block_size=4)
    for x, y in [(a.q, b.q), (a.k_pool, b.k_pool), (a.block_table, b.block_table)]:
        assert np.array_equal(x, y)


def test_unknown_storage_dtype_rejected():
    with pytest.raises(ValueError):
        inputs.to_storage(np.zeros(3), "fp8")
