"""The seeded generator: determinism, shapes, distributions, bf16 rounding."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.0039062, 3.4e38, 1e-40, 0.0, -0.0],
                                 np.float32)])
    ours = W.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_gqa_config_shapes(cfg):
    s = W.CONFIGS[cfg]
    lens = W.draw_seq_lens(s.batch, s.seq_len, s.seq_len_range, cfg)
    assert lens.shape == (s.batch,)
    if s.seq_len is not None:
        assert np.all(lens == s.seq_len)
    else:
        lo, hi = s.seq_len_range
        assert lens.min() >= lo and lens.max() <= hi


def test_small_config_bits_are_deterministic_and_distributed():
    a = W.make_gqa_config(1)
    b = W.make_gqa_config(1)
    assert a.q.dtype == np.float32 and a.k.shape == (1, 128, 2, 64)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    x = np.concatenate([a.k.ravel(), a.v.ravel()])
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05
    c = W.make_gqa_config(1, seed=1)
    assert not np.array_equal(a.k, c.k)


def test_config5_lengths_and_partial_generation():
    s = W.CONFIGS[5]
    lens = W.draw_seq_lens(s.batch, None, s.seq_len_range, 5)
    assert lens.min() >= 1 and lens.max() <= 8192
    # regenerating only a few sequences gives the same bits as the full draw
    small = W.make_gqa(4, 2, 2, 8, lens[:4] % 50 + 1, "bf16", cfg=5, max_seq_len=64)
    part = W.make_gqa(4, 2, 2, 8, lens[:4] % 50 + 1, "bf16", cfg=5, max_seq_len=64, only_seqs=[2])
    L2 = int(lens[2] % 50 + 1)
    assert np.array_equal(small.k[2, :L2], part.k[2, :L2])
    assert np.array_equal(small.v[2, :L2], part.v[2, :L2])
    assert np.array_equal(small.q, part.q)


def test_nan_padding_marks_rows_past_the_length():
    g = W.make_gqa(2, 4, 2, 8, [3, 5], "bf16", max_seq_len=8, pad_value=float("nan"))
    k = W.bf16_to_f32(g.k)
    assert np.isnan(k[0, 3:]).all() and np.isfinite(k[0, :3]).all()
    assert np.isnan(k[1, 5:]).all() and np.isfinite(k[1, :5]).all()
    m = W.make_mla(2, 16, [2, 4], max_seq_len=6, pad_value=float("nan"))
    c = W.bf16_to_f32(m.cache)
    assert np.isnan(c[0, 2:]).all() and np.isfinite(c[0, :2]).all()


def test_mla_weights_have_variance_one_over_512():
    m = W.make_mla(1, 16, [4], max_seq_len=4)
    w = W.bf16_to_f32(m.w_uk).astype(np.float64)
    assert m.w_uk.shape == (16, 512, 128) and m.w_uv.shape == (16, 512, 128)
    assert abs(w.var() * 512 - 1) < 0.02
    assert m.cache.shape == (1, 4, 576)
    assert m.scale == pytest.approx(1 / np.sqrt(192))


def test_mla_config4_lengths_in_range():
    s = W.CONFIGS[4]
    lens = W.draw_seq_lens(s.batch, None, s.seq_len_range, 4)
    assert lens.min() >= 16384 and lens.max() <= 32768


def test_paginate_places_every_row_and_fills_the_rest():
    lens = [5, 0, 33, 16]
    table, n = W.make_block_table(lens, 16, seed=4, spare_pages=2)
    assert n == 1 + 0 + 3 + 1 + 2
    used = table[table >= 0]
    assert len(set(used.tolist())) == len(used) and used.max() < n      # pages are distinct and in the pool
    assert np.all(table[1] == -1) and np.all(table[0, 1:] == -1)
    cache = np.arange(4 * 40 * 3, dtype=np.int64).reshape(4, 40, 3)
    pool = W.paginate(cache, lens, table, n, 16, -7)
    for b, L in enumerate(lens):
        for t in range(L):
            np.testing.assert_array_equal(pool[table[b, t // 16], t % 16], cache[b, t])
    assert (pool == -7).all(axis=-1).sum() == n * 16 - sum(lens)       # everything else is fill
