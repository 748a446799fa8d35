"""Pin the fp64 oracle (oracle/attention.py) to things other than itself.

Each pin is chosen so a plausible mistake in the oracle fails at least one:
  * scalar brute force with math.fsum on tiny inputs (vectorisation / axis errors);
  * closed forms: L=1, identical keys, a dominant key, V = ones (rows sum to 1);
  * one-hot V per KV head (which KV head each query head reads);
  * torch's scaled_dot_product_attention in float64 (an independent library routine),
    for MHA, for GQA (enable_gqa) and for explicitly up-projected MLA;
  * absorbed MLA == explicit MLA (associativity);
  * MLA with identity up-projections and no RoPE == MQA (cross-pins the two paths);
  * split-KV merge of any partition (including empty chunks) == unsplit result.
The planted-mistake tests at the end re-run some pins against a deliberately
broken copy of an oracle step and check that the pin then fails.
"""
import math

import numpy as np
import pytest
import torch

import oracle.attention as OA
from oracle.attention import (combine_ref, gqa_decode_ref, mla_absorbed_ref,
                              mla_explicit_ref)

RNG = np.random.default_rng(1234)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------------------
# brute force
# ----------------------------------------------------------------------------

def brute_gqa(q, k, v, seq_lens, scale):
    """Scalar loops with exact-ish summation; independent of numpy vector ops."""
    B, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hq):
            kv = h // g
            if L == 0:
                continue
            s = [scale * math.fsum(float(q[b, h, i]) * float(k[b, j, kv, i]) for i in range(D))
                 for j in range(L)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            lse[b, h] = m + math.log(z)
            for i in range(D):
                out[b, h, i] = math.fsum(e[j] / z * float(v[b, j, kv, i]) for j in range(L))
    return out, lse


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 2), (8, 1), (6, 3), (3, 1)])
@pytest.mark.parametrize("L", [1, 2, 5, 8])
def test_gqa_brute_force(Hq, Hkv, L):
    rng = np.random.default_rng([Hq, Hkv, L])
    B, D = 2, 5
    q = rand(B, Hq, D, rng=rng)
    k = rand(B, 8, Hkv, D, rng=rng)
    v = rand(B, 8, Hkv, D, rng=rng)
    lens = np.array([L, max(1, L - 1)])
    o, l = gqa_decode_ref(q, k, v, lens, 0.7)
    ob, lb = brute_gqa(q, k, v, lens, 0.7)
    np.testing.assert_allclose(o, ob, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l, lb, rtol=1e-13, atol=1e-13)


def brute_mla(q_nope, q_rope, cache, seq_lens, w_uk, w_uv, scale, d_c):
    """Scalar loops of the literal (up-projected) MLA formula."""
    B, H, dn = q_nope.shape
    dr = q_rope.shape[2]
    dv = w_uv.shape[2]
    out = np.zeros((B, H, dv))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(H):
            s = []
            for j in range(L):
                kc = [math.fsum(cache[b, j, c] * w_uk[h, c, e] for c in range(d_c)) for e in range(dn)]
                dot = math.fsum([q_nope[b, h, e] * kc[e] for e in range(dn)] +
                                [q_rope[b, h, r] * cache[b, j, d_c + r] for r in range(dr)])
                s.append(scale * dot)
            m = max(s)
            e_ = [math.exp(x - m) for x in s]
            z = math.fsum(e_)
            lse[b, h] = m + math.log(z)
            for e in range(dv):
                vcol = [math.fsum(cache[b, j, c] * w_uv[h, c, e] for c in range(d_c)) for j in range(L)]
                out[b, h, e] = math.fsum(e_[j] / z * vcol[j] for j in range(L))
    return out, lse


@pytest.mark.parametrize("H,d_c,d_r,L", [(1, 4, 0, 1), (2, 4, 2, 3), (4, 8, 2, 8), (2, 8, 0, 5)])
def test_mla_brute_force(H, d_c, d_r, L):
    rng = np.random.default_rng([H, d_c, d_r, L, 7])
    B, dn, dv = 2, 3, 4
    qn, qr = rand(B, H, dn, rng=rng), rand(B, H, d_r, rng=rng)
    cache = rand(B, 8, d_c + d_r, rng=rng)
    wuk, wuv = rand(H, d_c, dn, rng=rng), rand(H, d_c, dv, rng=rng)
    lens = np.array([L, 1])
    sc = 1.0 / math.sqrt(dn + d_r)
    ob, lb = brute_mla(qn, qr, cache, lens, wuk, wuv, sc, d_c)
    for fn in (mla_absorbed_ref, mla_explicit_ref):
        o, l = fn(qn, qr, cache, lens, wuk, wuv, sc, kv_lora_rank=d_c)
        np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l, lb, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# closed forms and invariants
# ----------------------------------------------------------------------------

def test_L1_returns_the_single_value_row():
    q, k, v = rand(3, 4, 8), rand(3, 2, 2, 8), rand(3, 2, 2, 8)
    o, l = gqa_decode_ref(q, k, v, [1, 1, 1], 0.5)
    for b in range(3):
        for h in range(4):
            np.testing.assert_allclose(o[b, h], v[b, 0, h // 2], rtol=0, atol=1e-15)
            assert l[b, h] == pytest.approx(0.5 * float(q[b, h] @ k[b, 0, h // 2]), abs=1e-14)


def test_identical_keys_give_mean_of_values():
    B, L, D = 2, 7, 16
    q = rand(B, 2, D)
    krow = rand(B, 1, 1, D)
    k = np.repeat(krow, L, axis=1)
    v = rand(B, L, 1, D)
    o, l = gqa_decode_ref(q, k, v, [L, L], 0.25)
    for b in range(B):
        for h in range(2):
            np.testing.assert_allclose(o[b, h], v[b, :, 0].mean(axis=0), atol=1e-14)
            s = 0.25 * float(q[b, h] @ krow[b, 0, 0])
            assert l[b, h] == pytest.approx(s + math.log(L), abs=1e-13)


def test_dominant_key_selects_its_value():
    D, L = 8, 6
    q = np.zeros((1, 1, D)); q[0, 0, 0] = 1.0
    k = np.zeros((1, L, 1, D)); k[0, 3, 0, 0] = 50.0
    v = rand(1, L, 1, D)
    o, l = gqa_decode_ref(q, k, v, [L], 1.0)
    # the other five weights are each exp(-50) relative to the dominant one
    np.testing.assert_allclose(o[0, 0], v[0, 3, 0], rtol=0, atol=10 * L * math.exp(-50))
    assert l[0, 0] == pytest.approx(50.0 + math.log(1 + 5 * math.exp(-50)), abs=1e-14)


def test_softmax_rows_sum_to_one_and_weights_in_unit_interval():
    B, Hq, Hkv, D, L = 2, 4, 2, 8, 8
    q, k = rand(B, Hq, D), rand(B, L, Hkv, D) * 3
    ones = np.ones((B, L, Hkv, D))
    o, _ = gqa_decode_ref(q, k, ones, [L, 5], 0.9)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)
    # one-hot V per token exposes each softmax weight p_j as an output element
    eye = np.zeros((B, L, Hkv, D))
    for j in range(L):
        eye[:, j, :, j] = 1.0
    p, lse = gqa_decode_ref(q, k, eye, [L, 5], 0.9)
    assert (p >= 0).all() and (p <= 1).all()
    np.testing.assert_allclose(p.sum(axis=2), 1.0, atol=1e-14)
    assert np.all(p[1, :, 5:] == 0)      # tokens past the length get no weight
    # and each weight equals exp(s_j - lse)
    for b, Lb in enumerate([L, 5]):
        for h in range(Hq):
            s = 0.9 * k[b, :Lb, h // 2] @ q[b, h]
            np.testing.assert_allclose(p[b, h, :Lb], np.exp(s - lse[b, h]), atol=1e-14)


def test_token_permutation_invariance():
    B, Hq, Hkv, D, L = 1, 4, 1, 8, 8
    q, k, v = rand(B, Hq, D), rand(B, L, Hkv, D), rand(B, L, Hkv, D)
    perm = RNG.permutation(L)
    o1, l1 = gqa_decode_ref(q, k, v, [L], 0.3)
    o2, l2 = gqa_decode_ref(q, k[:, perm], v[:, perm], [L], 0.3)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


def test_empty_sequence():
    q, k, v = rand(2, 4, 8), rand(2, 3, 2, 8), rand(2, 3, 2, 8)
    o, l = gqa_decode_ref(q, k, v, [0, 3], 0.5)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    assert np.all(np.isfinite(l[1]))


def head_mapping_expected(Hq, Hkv):
    """V rows one-hot on the KV-head index: output of head h must be e_{h // g}."""
    g = Hq // Hkv
    exp = np.zeros((Hq, max(Hkv, 2)))
    for h in range(Hq):
        exp[h, h // g] = 1.0
    return exp


def check_head_mapping(fn, Hq, Hkv):
    D, L = max(Hkv, 2), 5
    q, k = rand(1, Hq, D), rand(1, L, Hkv, D)
    v = np.zeros((1, L, Hkv, D))
    for kv in range(Hkv):
        v[0, :, kv, kv] = 1.0
    o, _ = fn(q, k, v, [L], 0.5)
    np.testing.assert_allclose(o[0], head_mapping_expected(Hq, Hkv), atol=1e-14)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (32, 8), (8, 8), (8, 1), (6, 3)])
def test_head_mapping_one_hot(Hq, Hkv):
    # 8 query heads, 2 KV heads: heads 0-3 read KV 0, heads 4-7 read KV 1
    # (kakack.github.io section 4; shippingwang.com section 7.3)
    check_head_mapping(gqa_decode_ref, Hq, Hkv)


# ----------------------------------------------------------------------------
# torch SDPA in float64 (library routine)
# ----------------------------------------------------------------------------

def sdpa(q, k, v, scale, gqa=False):
    """q [Hq, D], k/v [L, Hkv, D] -> [Hq, Dv] via torch float64 SDPA."""
    tq = torch.from_numpy(np.ascontiguousarray(q))[None, :, None, :]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale, enable_gqa=gqa)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 64), (32, 8, 128), (8, 1, 32), (12, 4, 16)])
def test_gqa_vs_torch_sdpa(Hq, Hkv, D):
    B, L = 3, 37
    q, k, v = rand(B, Hq, D), rand(B, L, Hkv, D), rand(B, L, Hkv, D)
    lens = [37, 1, 20]
    sc = 1 / math.sqrt(D)
    o, _ = gqa_decode_ref(q, k, v, lens, sc)
    for b, Lb in enumerate(lens):
        ot = sdpa(q[b], k[b, :Lb], v[b, :Lb], sc, gqa=Hq != Hkv)
        np.testing.assert_allclose(o[b], ot, rtol=1e-12, atol=1e-13)


def test_mla_explicit_vs_torch_sdpa_full_dims():
    # DeepSeek-V3 per-head dimensions: d_c 512, rope 64, nope 128, v 128
    H, L, d_c, d_r, dn, dv = 4, 24, 512, 64, 128, 128
    qn, qr = rand(1, H, dn), rand(1, H, d_r)
    cache = rand(1, L, d_c + d_r)
    wuk, wuv = rand(H, d_c, dn) / math.sqrt(512), rand(H, d_c, dv) / math.sqrt(512)
    sc = 1 / math.sqrt(192)
    o, _ = mla_explicit_ref(qn, qr, cache, [L], wuk, wuv, sc)
    tc = torch.from_numpy(cache[0])
    for h in range(H):
        kc = tc[:, :d_c] @ torch.from_numpy(wuk[h])                  # [L, 128]
        kfull = torch.cat([kc, tc[:, d_c:]], dim=1)                   # [L, 192]
        vfull = tc[:, :d_c] @ torch.from_numpy(wuv[h])                # [L, 128]
        qfull = torch.cat([torch.from_numpy(qn[0, h]), torch.from_numpy(qr[0, h])])
        ot = torch.nn.functional.scaled_dot_product_attention(
            qfull[None, None, None], kfull[None, None], vfull[None, None], scale=sc)
        np.testing.assert_allclose(o[0, h], ot[0, 0, 0].numpy(), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# MLA associativity and the MQA special case
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("H", [1, 2, 4])
@pytest.mark.parametrize("d_c", [4, 8])
@pytest.mark.parametrize("d_r", [0, 2])
def test_mla_absorbed_equals_explicit_tiny(H, d_c, d_r):
    rng = np.random.default_rng([H, d_c, d_r])
    B, Lmax, dn, dv = 2, 8, 3, 5
    qn, qr = rand(B, H, dn, rng=rng), rand(B, H, d_r, rng=rng)
    cache = rand(B, Lmax, d_c + d_r, rng=rng)
    wuk, wuv = rand(H, d_c, dn, rng=rng), rand(H, d_c, dv, rng=rng)
    lens = [8, 3]
    sc = 1 / math.sqrt(dn + d_r)
    oa, la = mla_absorbed_ref(qn, qr, cache, lens, wuk, wuv, sc, kv_lora_rank=d_c)
    oe, le = mla_explicit_ref(qn, qr, cache, lens, wuk, wuv, sc, kv_lora_rank=d_c)
    np.testing.assert_allclose(oa, oe, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(la, le, rtol=1e-12, atol=1e-12)


def test_mla_absorbed_equals_explicit_full_rows():
    H, L = 4, 16
    qn, qr = rand(2, H, 128), rand(2, H, 64)
    cache = rand(2, L, 576)
    wuk, wuv = rand(H, 512, 128) / math.sqrt(512), rand(H, 512, 128) / math.sqrt(512)
    sc = 1 / math.sqrt(192)
    oa, la = mla_absorbed_ref(qn, qr, cache, [16, 9], wuk, wuv, sc)
    oe, le = mla_explicit_ref(qn, qr, cache, [16, 9], wuk, wuv, sc)
    np.testing.assert_allclose(oa, oe, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(la, le, rtol=1e-12, atol=1e-12)


def test_mla_with_identity_projections_is_mqa():
    # GQA/MQA is MLA whose up-projections are 0/1 selection matrices
    # (arganzheng.life section 4.7): identity W_UK = W_UV, no RoPE, K = V = C.
    B, H, d, L = 2, 4, 8, 6
    qn, qr = rand(B, H, d), np.zeros((B, H, 0))
    cache = rand(B, L, d)
    eye = np.broadcast_to(np.eye(d), (H, d, d)).copy()
    o1, l1 = mla_absorbed_ref(qn, qr, cache, [6, 2], eye, eye, 0.4, kv_lora_rank=d)
    kv = cache[:, :, None, :]
    o2, l2 = gqa_decode_ref(qn, kv, kv, [6, 2], 0.4)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


# ----------------------------------------------------------------------------
# split-KV combine
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("cuts", [[0, 8], [0, 3, 8], [0, 0, 5, 5, 8], [0, 1, 2, 3, 4, 5, 6, 7, 8],
                                  [0, 8, 8]])
def test_combine_any_partition_equals_unsplit(cuts):
    B, Hq, Hkv, D, L = 2, 4, 2, 8, 8
    q, k, v = rand(B, Hq, D), rand(B, L, Hkv, D), rand(B, L, Hkv, D)
    o, l = gqa_decode_ref(q, k, v, [L, L], 0.35)
    po, pl = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        oo, ll = gqa_decode_ref(q, k[:, a:b], v[:, a:b], [b - a, b - a], 0.35)
        po.append(oo)
        pl.append(ll)
    oc, lc = combine_ref(np.stack(po), np.stack(pl))
    np.testing.assert_allclose(oc, o, atol=1e-13)
    np.testing.assert_allclose(lc, l, atol=1e-13)


def test_combine_all_empty_and_nan_in_empty_split():
    po = np.full((3, 2, 4), np.nan)
    pl = np.full((3, 2), -np.inf)
    o, l = combine_ref(po, pl)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    # an empty split's (garbage) output never leaks into the result
    po2 = rand(2, 2, 4)
    po2[1] = np.nan
    pl2 = np.stack([rand(2), np.full(2, -np.inf)])
    o2, l2 = combine_ref(po2, pl2)
    np.testing.assert_allclose(o2, po2[0], atol=0)
    np.testing.assert_allclose(l2, pl2[0], atol=0)


# ----------------------------------------------------------------------------
# planted mistakes: the pins above must catch a broken oracle
# ----------------------------------------------------------------------------

def test_planted_interleaved_head_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(OA, "kv_head_of", lambda h, nq, nkv: h % nkv)
    with pytest.raises(AssertionError):
        check_head_mapping(OA.gqa_decode_ref, 8, 2)


def test_planted_wrong_mla_scale_is_caught(monkeypatch):
    real = OA.mla_absorbed_ref

    def wrong(qn, qr, cache, lens, wuk, wuv, scale, kv_lora_rank=512):
        return real(qn, qr, cache, lens, wuk, wuv, 1 / math.sqrt(576), kv_lora_rank)

    H, L = 2, 6
    qn, qr, cache = rand(1, H, 128), rand(1, H, 64), rand(1, L, 576)
    wuk, wuv = rand(H, 512, 128) / 22.6, rand(H, 512, 128) / 22.6
    oe, _ = mla_explicit_ref(qn, qr, cache, [L], wuk, wuv, 1 / math.sqrt(192))
    ow, _ = wrong(qn, qr, cache, [L], wuk, wuv, 1 / math.sqrt(192))
    with pytest.raises(AssertionError):
        np.testing.assert_allclose(ow, oe, rtol=1e-12, atol=1e-12)


def test_planted_transposed_wuk_is_caught():
    # absorbing with W_UK[h] used the wrong way round breaks associativity
    H, d_c, dn, L = 2, 6, 6, 5
    qn, qr, cache = rand(1, H, dn), rand(1, H, 2), rand(1, L, d_c + 2)
    wuk, wuv = rand(H, d_c, dn), rand(H, d_c, 3)
    sc = 0.3
    oe, _ = mla_explicit_ref(qn, qr, cache, [L], wuk, wuv, sc, kv_lora_rank=d_c)
    ow, _ = mla_absorbed_ref(qn, qr, cache, [L], wuk.transpose(0, 2, 1), wuv, sc, kv_lora_rank=d_c)
    with pytest.raises(AssertionError):
        np.testing.assert_allclose(ow, oe, rtol=1e-9, atol=1e-9)


def test_planted_dropped_empty_split_guard_is_caught():
    # merging that multiplies an empty split's NaN output by its zero weight
    po = rand(2, 1, 4)
    po[1] = np.nan
    pl = np.stack([rand(1), np.full(1, -np.inf)])
    w = np.exp(pl - pl.max(axis=0))
    naive = np.einsum("sb,sbd->bd", w / w.sum(axis=0), po)
    assert np.isnan(naive).any()
    o, _ = combine_ref(po, pl)
    assert np.isfinite(o).all()


# ----------------------------------------------------------------------------
# paged caches (arganzheng.life section 6.1: blocks of page_size tokens in a
# shared pool, found through a per-sequence block table)
# ----------------------------------------------------------------------------

import workloads as W
from oracle.attention import gqa_decode_paged_ref, mla_absorbed_paged_ref


def brute_paged_gqa(q, k_pool, v_pool, table, ps, seq_lens, scale):
    """Scalar loops that look every row up in the block table themselves."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            rows = [(int(table[b][t // ps]), t % ps) for t in range(int(seq_lens[b]))]
            if not rows:
                continue
            s = [scale * math.fsum(q[b, h, d] * k_pool[p, r, kv, d] for d in range(D)) for p, r in rows]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            lse[b, h] = m + math.log(z)
            for d in range(D):
                out[b, h, d] = math.fsum(w[j] * v_pool[p, r, kv, d] for j, (p, r) in enumerate(rows)) / z
    return out, lse


def paged_case(B, Hq, Hkv, D, lens, ps, seed, spare=3):
    rng = np.random.default_rng(seed)
    L = max(1, max(lens))
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, L, Hkv, D))
    v = rng.standard_normal((B, L, Hkv, D))
    table, n = W.make_block_table(lens, ps, seed=seed, spare_pages=spare)
    kp = W.paginate(k, lens, table, n, ps, np.nan)
    vp = W.paginate(v, lens, table, n, ps, np.nan)
    return q, k, v, kp, vp, table


@pytest.mark.parametrize("ps,lens", [(2, [5, 1, 0, 4]), (4, [9, 3, 8]), (1, [3, 2])])
def test_paged_gqa_brute_force(ps, lens):
    q, k, v, kp, vp, table = paged_case(len(lens), 4, 2, 3, lens, ps, seed=5)
    o, l = gqa_decode_paged_ref(q, kp, vp, table, ps, lens, 0.7)
    bo, bl = brute_paged_gqa(q, kp, vp, table, ps, lens, 0.7)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isfinite(l), np.isfinite(bl))
    np.testing.assert_allclose(l[np.isfinite(l)], bl[np.isfinite(bl)], rtol=1e-12, atol=1e-12)


def test_paged_gqa_equals_contiguous_and_ignores_physical_order():
    lens = [37, 16, 0, 1, 64]
    q, k, v, kp, vp, table = paged_case(5, 8, 2, 16, lens, 16, seed=6)
    o, l = gqa_decode_paged_ref(q, kp, vp, table, 16, lens, 0.25)
    ro, rl = gqa_decode_ref(q, k, v, lens, 0.25)     # the contiguous cache the pool was built from
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(l, rl)
    # another physical placement of the same pages: the same result
    t2, n2 = W.make_block_table(lens, 16, seed=99, spare_pages=5)
    o2, l2 = gqa_decode_paged_ref(q, W.paginate(k, lens, t2, n2, 16, np.nan), W.paginate(v, lens, t2, n2, 16, np.nan),
                                  t2, 16, lens, 0.25)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_paged_mla_equals_contiguous():
    rng = np.random.default_rng(8)
    B, H, dc, dr, dn = 3, 4, 8, 2, 5
    lens = [20, 0, 7]
    L = 20
    qn, qr = rng.standard_normal((B, H, dn)), rng.standard_normal((B, H, dr))
    cache = rng.standard_normal((B, L, dc + dr))
    wuk, wuv = rng.standard_normal((H, dc, dn)), rng.standard_normal((H, dc, 6))
    table, n = W.make_block_table(lens, 4, seed=3)
    pool = W.paginate(cache, lens, table, n, 4, np.nan)
    o, l = mla_absorbed_paged_ref(qn, qr, pool, table, 4, lens, wuk, wuv, 0.3, kv_lora_rank=dc)
    ro, rl = mla_absorbed_ref(qn, qr, cache, lens, wuk, wuv, 0.3, kv_lora_rank=dc)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(l, rl)


def test_planted_reversed_page_order_is_caught(monkeypatch):
    def broken(pool, table_row, page_size, seq_len):
        n_blocks = -(-int(seq_len) // page_size)
        pages = np.asarray(table_row[:n_blocks], dtype=np.int64)[::-1]   # blocks in the wrong order
        rows = pool[pages].reshape((n_blocks * page_size,) + pool.shape[2:])
        return rows[:seq_len]
    monkeypatch.setattr(OA, "paged_rows_ref", broken)
    q, k, v, kp, vp, table = paged_case(2, 4, 2, 3, [9, 8], 4, seed=5, spare=0)
    o, l = OA.gqa_decode_paged_ref(q, kp, vp, table, 4, [9, 8], 0.7)
    bo, bl = brute_paged_gqa(q, kp, vp, table, 4, [9, 8], 0.7)
    assert not (np.all(np.isfinite(o)) and np.allclose(o, bo, rtol=1e-9))


# ----------------------------------------------------------------------------
# FP8 (E4M3) caches ("Attention variants and KV cache", section 6.3)
# ----------------------------------------------------------------------------

import oracle.fp8 as OF
from oracle.fp8 import dequantize_ref, e4m3_to_float, gqa_decode_fp8_ref


def brute_e4m3(c: int) -> float:
    """One code, from the OCP E4M3 definition, by scalar arithmetic."""
    sign = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return math.nan
    return sign * (math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10))


def test_e4m3_decoder_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_to_float(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).sum() == 2
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))     # -0 for 0x80


def test_e4m3_defining_values_and_structure():
    # OCP 8-bit floating point specification, E4M3: bias 7, largest normal
    # 448 = 1.75 * 2^8, smallest normal 2^-6, smallest subnormal 2^-9
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xC0: -2.0, 0xFE: -448.0}
    for c, v in fixed.items():
        assert e4m3_to_float(np.array([c], np.uint8))[0] == v, hex(c)
    codes = np.arange(256, dtype=np.uint8)
    val = e4m3_to_float(codes)
    assert all(val[c] == brute_e4m3(c) or (math.isnan(val[c]) and math.isnan(brute_e4m3(c)))
               for c in range(256))
    assert np.all(np.diff(val[:127]) > 0)                     # increasing over 0x00..0x7E
    assert np.array_equal(val[128:255], -val[:127])           # sign symmetry
    assert np.isnan(val[0x7F]) and np.isnan(val[0xFF])


def test_planted_fnuz_bias_is_caught(monkeypatch):
    # the other common E4M3 variant has bias 8; the pins above must notice
    monkeypatch.setattr(OF, "E4M3_BIAS", 8)
    with pytest.raises(AssertionError):
        test_e4m3_decoder_matches_torch_for_every_code()


def _fp8_inputs(B, Hq, Hkv, D, lens, seed):
    rng = np.random.default_rng(seed)
    L = max(lens)
    codes = lambda: rng.integers(0, 256, (B, L, Hkv, D)).astype(np.uint8)
    k, v = codes(), codes()
    for x in (k, v):                                  # no NaN codes
        x[(x & 0x7F) == 0x7F] = 0x38
    ks = rng.uniform(0.01, 0.05, (B, L, Hkv))
    vs = rng.uniform(0.5, 2.0, (B, L, Hkv))
    q = rng.standard_normal((B, Hq, D))
    return q, k, v, ks, vs


def brute_gqa_fp8(q, k, v, ks, vs, seq_lens, scale):
    """Scalar loops: decode each code, scale it, attend with math.fsum."""
    B, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hq):
            kv = h // g
            if L == 0:
                continue
            s = [scale * math.fsum(q[b, h, i] * brute_e4m3(int(k[b, j, kv, i])) * ks[b, j, kv]
                                   for i in range(D)) for j in range(L)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            lse[b, h] = m + math.log(z)
            for i in range(D):
                out[b, h, i] = math.fsum(e[j] / z * brute_e4m3(int(v[b, j, kv, i])) * vs[b, j, kv]
                                         for j in range(L))
    return out, lse


@pytest.mark.parametrize("Hq,Hkv,lens", [(4, 2, [3, 1]), (6, 3, [5, 0]), (2, 2, [4, 4])])
def test_fp8_gqa_brute_force(Hq, Hkv, lens):
    q, k, v, ks, vs = _fp8_inputs(len(lens), Hq, Hkv, 8, lens, seed=sum(lens) + Hq)
    o, l = gqa_decode_fp8_ref(q, k, v, ks, vs, lens, 0.3)
    bo, bl = brute_gqa_fp8(q, k, v, ks, vs, lens, 0.3)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, bl, rtol=1e-12, atol=1e-12)


def test_fp8_gqa_scale_closed_forms():
    q, k, v, ks, vs = _fp8_inputs(2, 4, 2, 16, [6, 3], seed=5)
    lens = [6, 3]
    # a zero key scale makes every score 0: the output is the mean of the
    # dequantized values and lse = ln L
    o, l = gqa_decode_fp8_ref(q, k, v, np.zeros_like(ks), vs, lens, 0.5)
    for b, L in enumerate(lens):
        vals = dequantize_ref(v[b, :L], vs[b, :L])            # [L, Hkv, D]
        for h in range(4):
            np.testing.assert_allclose(o[b, h], vals[:, h // 2].mean(axis=0), rtol=1e-12)
            assert abs(l[b, h] - math.log(L)) < 1e-12
    # doubling every value scale doubles the output and leaves lse alone
    o1, l1 = gqa_decode_fp8_ref(q, k, v, ks, vs, lens, 0.5)
    o2, l2 = gqa_decode_fp8_ref(q, k, v, ks, 2 * vs, lens, 0.5)
    np.testing.assert_allclose(o2, 2 * o1, rtol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-12)
    # a key scale that is huge for one token makes that token dominant
    ks2 = ks.copy()
    ks2[0, 2, :] = 1e4
    k2 = k.copy()
    k2[0, 2] = 0x38                                           # every element 1.0
    q2 = np.abs(q)                                            # positive dot products
    o3, _ = gqa_decode_fp8_ref(q2, k2, v, ks2, vs, lens, 0.5)
    for h in range(4):
        np.testing.assert_allclose(o3[0, h], dequantize_ref(v[0, 2], vs[0, 2])[h // 2], rtol=1e-9)


def test_planted_swapped_kv_scales_are_caught():
    q, k, v, ks, vs = _fp8_inputs(2, 4, 2, 8, [3, 2], seed=9)
    bo, bl = brute_gqa_fp8(q, k, v, ks, vs, [3, 2], 0.4)
    o, l = gqa_decode_fp8_ref(q, k, v, vs, ks, [3, 2], 0.4)   # the mistake
    assert not np.allclose(o, bo, rtol=1e-3)


def test_fp8_workload_codes_round_trip():
    # the generator's codes decode to within half an E4M3 step of the drawn
    # values, relative to the row's scale (round to nearest)
    inp = W.make_gqa_fp8(2, 4, 2, 64, [7, 3], seed=4)
    for b, L in enumerate(inp.seq_lens):
        r = np.random.default_rng([4, 0, 2, b])
        kf = r.standard_normal((L, 2, 64), dtype=np.float32)
        deq = dequantize_ref(inp.k[b, :L], inp.k_scale[b, :L])
        rel = np.abs(deq - kf) / np.abs(kf).max(axis=-1, keepdims=True)
        assert rel.max() <= 2.0 ** -4 * 1.0001
        assert np.all(np.abs(e4m3_to_float(inp.k[b, :L])) <= 448)
    assert np.all(inp.k[0, 7:] == W.FP8_NAN_CODE) and np.isnan(inp.v_scale[1, 3:]).all()


# ----------------------------------------------------------------------------
# MLA over an E4M3 latent cache, nope and rope ranges scaled apart
# ("Attention variants and KV cache", sections 4.8 and 6.3)
# ----------------------------------------------------------------------------

def _mla_fp8_inputs(B, H, d_c, d_r, d_n, lens, seed):
    rng = np.random.default_rng(seed)
    L = max(lens)
    codes = rng.integers(0, 256, (B, L, d_c + d_r)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                 # no NaN codes
    sn = rng.uniform(0.002, 0.01, (B, L))                 # the nope range: small values
    sr = rng.uniform(0.05, 0.2, (B, L))                   # the rope range: larger ones
    qn = rng.standard_normal((B, H, d_n))
    qr = rng.standard_normal((B, H, d_r))
    wuk = rng.standard_normal((H, d_c, d_n)) / math.sqrt(d_c)
    wuv = rng.standard_normal((H, d_c, 5)) / math.sqrt(d_c)
    return qn, qr, codes, sn, sr, wuk, wuv


def brute_mla_fp8(qn, qr, codes, sn, sr, seq_lens, wuk, wuv, scale, d_c):
    """Scalar loops with math.fsum: decode every code, scale it by its
    range's scale, absorb, attend the latent rows, project."""
    B, H, d_n = qn.shape
    d_v = wuv.shape[2]
    out = np.zeros((B, H, d_v))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        rows = [[brute_e4m3(int(codes[b, j, c])) * (sn[b, j] if c < d_c else sr[b, j])
                 for c in range(codes.shape[2])] for j in range(L)]
        for h in range(H):
            qt = [math.fsum(wuk[h, c, e] * qn[b, h, e] for e in range(d_n)) for c in range(d_c)]
            qh = qt + list(qr[b, h])
            s = [scale * math.fsum(qh[c] * rows[j][c] for c in range(len(qh))) for j in range(L)]
            m = max(s)
            ex = [math.exp(x - m) for x in s]
            z = math.fsum(ex)
            lse[b, h] = m + math.log(z)
            ot = [math.fsum(ex[j] / z * rows[j][c] for j in range(L)) for c in range(d_c)]
            for e in range(d_v):
                out[b, h, e] = math.fsum(ot[c] * wuv[h, c, e] for c in range(d_c))
    return out, lse


@pytest.mark.parametrize("H,d_c,d_r,lens", [(2, 8, 4, [3, 1]), (3, 4, 2, [5, 0]), (1, 8, 0, [4])])
def test_fp8_mla_brute_force(H, d_c, d_r, lens):
    qn, qr, codes, sn, sr, wuk, wuv = _mla_fp8_inputs(len(lens), H, d_c, d_r, 3, lens, seed=H + d_c)
    o, l = OF.mla_absorbed_fp8_ref(qn, qr, codes, sn, sr, lens, wuk, wuv, 0.4, kv_lora_rank=d_c)
    bo, bl = brute_mla_fp8(qn, qr, codes, sn, sr, lens, wuk, wuv, 0.4, d_c)
    np.testing.assert_allclose(o, bo, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(l, bl, rtol=1e-12, atol=1e-12)


def test_fp8_mla_ranges_scale_apart():
    qn, qr, codes, sn, sr, wuk, wuv = _mla_fp8_inputs(2, 3, 8, 4, 3, [6, 4], seed=17)
    lens = [6, 4]
    o1, l1 = OF.mla_absorbed_fp8_ref(qn, qr, codes, sn, sr, lens, wuk, wuv, 0.5, kv_lora_rank=8)
    # the rope scale multiplies only the rope part of every score: scaling it
    # by c equals scaling q_rope by c, and leaves the value (c_kv) alone
    o2, l2 = OF.mla_absorbed_fp8_ref(qn, qr, codes, sn, 3 * sr, lens, wuk, wuv, 0.5, kv_lora_rank=8)
    o3, l3 = OF.mla_absorbed_fp8_ref(qn, 3 * qr, codes, sn, sr, lens, wuk, wuv, 0.5, kv_lora_rank=8)
    np.testing.assert_allclose(o2, o3, rtol=1e-12)
    np.testing.assert_allclose(l2, l3, rtol=1e-12)
    # a zero rope scale removes the rope term: the same as q_rope = 0
    o4, l4 = OF.mla_absorbed_fp8_ref(qn, qr, codes, sn, 0 * sr, lens, wuk, wuv, 0.5, kv_lora_rank=8)
    o5, l5 = OF.mla_absorbed_fp8_ref(qn, 0 * qr, codes, sn, sr, lens, wuk, wuv, 0.5, kv_lora_rank=8)
    np.testing.assert_allclose(o4, o5, rtol=1e-12)
    np.testing.assert_allclose(l4, l5, rtol=1e-12)
    # zero nope and rope scales: every score 0, the rows are zero: lse = ln L, out = 0
    o6, l6 = OF.mla_absorbed_fp8_ref(qn, qr, codes, 0 * sn, 0 * sr, lens, wuk, wuv, 0.5, kv_lora_rank=8)
    np.testing.assert_allclose(l6, np.log(np.asarray(lens, float))[:, None] * np.ones((1, 3)), rtol=1e-13)
    assert np.all(o6 == 0)
    # the ranges are not interchangeable: one scale for the whole row differs
    o7, _ = OF.mla_absorbed_fp8_ref(qn, qr, codes, sn, sn, lens, wuk, wuv, 0.5, kv_lora_rank=8)
    assert not np.allclose(o7, o1, rtol=1e-3)


def test_fp8_mla_equals_bf16_oracle_on_dequantized_rows_and_explicit_path():
    from oracle.attention import mla_absorbed_ref, mla_explicit_ref
    qn, qr, codes, sn, sr, wuk, wuv = _mla_fp8_inputs(2, 4, 16, 8, 6, [7, 3], seed=23)
    lens = [7, 3]
    o, l = OF.mla_absorbed_fp8_ref(qn, qr, codes, sn, sr, lens, wuk, wuv, 0.3, kv_lora_rank=16)
    rows = OF.dequantize_mla_rows_ref(codes, sn, sr, kv_lora_rank=16)
    # the dequantized row is the pair of ranges, each at its own scale
    assert np.array_equal(rows[..., :16], e4m3_to_float(codes[..., :16]) * sn[..., None])
    assert np.array_equal(rows[..., 16:], e4m3_to_float(codes[..., 16:]) * sr[..., None])
    ob, lb = mla_absorbed_ref(qn, qr, rows, lens, wuk, wuv, 0.3, kv_lora_rank=16)
    oe, le = mla_explicit_ref(qn, qr, rows, lens, wuk, wuv, 0.3, kv_lora_rank=16)
    np.testing.assert_allclose(o, ob, rtol=1e-13)
    np.testing.assert_allclose(o, oe, rtol=1e-10)
    np.testing.assert_allclose(l, le, rtol=1e-12)


def test_fp8_mla_quantizer_scales_each_range_by_its_own_max():
    rng = np.random.default_rng(31)
    rows = np.concatenate([rng.standard_normal((5, 512)) * 1e-3, rng.standard_normal((5, 64)) * 300], axis=1)
    rows = rows.astype(np.float32)
    codes, sn, sr = OF.quantize_mla_rows_ref(rows)
    np.testing.assert_array_equal(sn, (np.abs(rows[:, :512]).max(axis=1) / np.float32(448)).astype(np.float32))
    np.testing.assert_array_equal(sr, (np.abs(rows[:, 512:]).max(axis=1) / np.float32(448)).astype(np.float32))
    back = OF.dequantize_mla_rows_ref(codes, sn, sr)
    # round to nearest: within half an E4M3 step (relative 2^-4) of each range's max
    for lo, hi, s in ((0, 512, sn), (512, 576, sr)):
        err = np.abs(back[:, lo:hi] - rows[:, lo:hi]) / (448 * s[:, None])
        assert err.max() <= 2.0 ** -4
    # with ranges this far apart one scale for the whole row would put the
    # nope values below E4M3's smallest subnormal (they become 0); the
    # separate scales keep them to 3 significant bits
    c1, s1 = OF.quantize_rows_ref(rows)
    one = OF.dequantize_ref(c1, s1)
    sep_err = np.abs(back[:, :512] - rows[:, :512]).max()
    one_err = np.abs(one[:, :512] - rows[:, :512]).max()
    assert sep_err * 10 < one_err


def test_fp8_mla_workload_codes_round_trip():
    # each range decodes to within half an E4M3 step of the drawn values,
    # relative to that range's own scale; padding rows are NaN
    inp = W.make_mla_fp8(2, 16, [9, 4], seed=6, max_seq_len=12, rope_std=50.0)
    for b, L in enumerate(inp.seq_lens):
        x = np.random.default_rng([6, 0, 2, b]).standard_normal((L, 576), dtype=np.float32)
        x[:, 512:] *= np.float32(50.0)
        back = OF.dequantize_mla_rows_ref(inp.cache[b, :L], inp.scale_nope[b, :L], inp.scale_rope[b, :L])
        for lo, hi, s in ((0, 512, inp.scale_nope[b, :L]), (512, 576, inp.scale_rope[b, :L])):
            assert (np.abs(back[:, lo:hi] - x[:, lo:hi]) / (448 * s[:, None])).max() <= 2.0 ** -4
    assert np.all(inp.cache[0, 9:] == W.FP8_NAN_CODE) and np.isnan(inp.scale_rope[1, 4:]).all()
    # same queries and weights as the bf16 generator
    m = W.make_mla(2, 16, [9, 4], seed=6, max_seq_len=12)
    assert np.array_equal(inp.q_nope, m.q_nope) and np.array_equal(inp.w_uv, m.w_uv)


def test_fp8_mla_paged_gathers_through_the_table():
    # per-row brute force through the table on a tiny pool, equality with the
    # contiguous reference on the same rows, invariance to the physical page
    # order, and a planted reversed page order caught
    qn, qr, codes, sn, sr, wuk, wuv = _mla_fp8_inputs(2, 3, 8, 4, 3, [7, 3], seed=41)
    lens = np.array([7, 3])
    ps = 2
    table, n_pages = W.make_block_table(lens, ps, seed=5, spare_pages=2)
    cp = W.paginate(codes, lens, table, n_pages, ps, W.FP8_NAN_CODE)
    snp = W.paginate(sn, lens, table, n_pages, ps, np.nan)
    srp = W.paginate(sr, lens, table, n_pages, ps, np.nan)
    for b, L in enumerate(lens):
        for t in range(L):
            pg, r = table[b, t // ps], t % ps
            assert np.array_equal(cp[pg, r], codes[b, t]) and snp[pg, r] == sn[b, t] and srp[pg, r] == sr[b, t]
    o, l = OF.mla_absorbed_fp8_paged_ref(qn, qr, cp, snp, srp, table, ps, lens, wuk, wuv, 0.4, kv_lora_rank=8)
    oc, lc = OF.mla_absorbed_fp8_ref(qn, qr, codes, sn, sr, lens, wuk, wuv, 0.4, kv_lora_rank=8)
    assert np.array_equal(o, oc) and np.array_equal(l, lc)
    table2, n2 = W.make_block_table(lens, ps, seed=99, spare_pages=0)
    cp2 = W.paginate(codes, lens, table2, n2, ps, W.FP8_NAN_CODE)
    o2, _ = OF.mla_absorbed_fp8_paged_ref(qn, qr, cp2, W.paginate(sn, lens, table2, n2, ps, np.nan),
                                          W.paginate(sr, lens, table2, n2, ps, np.nan), table2, ps, lens, wuk,
                                          wuv, 0.4, kv_lora_rank=8)
    assert np.array_equal(o2, oc)
    bad = table.copy()
    bad[0, :4] = bad[0, :4][::-1]
    ob, _ = OF.mla_absorbed_fp8_paged_ref(qn, qr, cp, snp, srp, bad, ps, lens, wuk, wuv, 0.4, kv_lora_rank=8)
    assert not np.allclose(ob[0], oc[0], rtol=1e-6)


# ----------------------------------------------------------------------------
# sliding window ("Attention variants and KV cache", section 5.3)
# ----------------------------------------------------------------------------

def brute_window(q, k, v, seq_lens, scale, w):
    """Scalar loops over an explicit mask: row j is seen iff L - w <= j < L."""
    B, Hq, D = q.shape
    g = Hq // k.shape[2]
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hq):
            js = [j for j in range(L) if j >= L - w]
            if not js:
                continue
            s = [scale * math.fsum(q[b, h, d] * k[b, j, h // g, d] for d in range(D)) for j in js]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            lse[b, h] = m + math.log(z)
            for d in range(D):
                out[b, h, d] = math.fsum(ei * v[b, j, h // g, d] for ei, j in zip(e, js)) / z
    return out, lse


@pytest.mark.parametrize("w", [1, 3, 7, 50])
def test_window_brute_force(w):
    q, k, v = rand(3, 4, 8), rand(3, 9, 2, 8), rand(3, 9, 2, 8)
    lens = [9, 4, 0]
    o, l = gqa_decode_ref(q, k, v, lens, 0.3, window=w)
    bo, bl = brute_window(q, k, v, lens, 0.3, w)
    np.testing.assert_allclose(o, bo, atol=1e-12)
    np.testing.assert_allclose(l, bl, atol=1e-12)


def test_window_closed_forms():
    q, k, v = rand(2, 4, 16), rand(2, 12, 2, 16), rand(2, 12, 2, 16)
    lens = [12, 5]
    full = gqa_decode_ref(q, k, v, lens, 0.25)
    for w in (12, 13, 1000):          # a window that holds every row changes nothing
        o, l = gqa_decode_ref(q, k, v, lens, 0.25, window=w)
        np.testing.assert_array_equal(o[0], full[0][0])
    o, l = gqa_decode_ref(q, k, v, lens, 0.25, window=1)      # only the newest row
    for b, L in enumerate(lens):
        for h in range(4):
            np.testing.assert_allclose(o[b, h], v[b, L - 1, h // 2], atol=1e-15)
            np.testing.assert_allclose(l[b, h], 0.25 * q[b, h] @ k[b, L - 1, h // 2], atol=1e-12)
    # shifted cache: the window over rows [L - w, L) == full attention over those rows at 0..w
    w = 4
    ks, vs = k[:, 12 - w:].copy(), v[:, 12 - w:].copy()
    o, l = gqa_decode_ref(q[:1], k[:1], v[:1], [12], 0.25, window=w)
    fo, fl = gqa_decode_ref(q[:1], ks[:1], vs[:1], [w], 0.25)
    np.testing.assert_allclose(o, fo, atol=1e-13)
    np.testing.assert_allclose(l, fl, atol=1e-13)


def test_window_sees_at_most_w_rows():
    # one-hot values by position make the output the softmax weights
    L, w = 10, 4
    q, k = rand(1, 1, 16), rand(1, L, 1, 16)
    v = np.zeros((1, L, 1, 16))
    for j in range(L):
        v[0, j, 0, j] = 1.0
    o, _ = gqa_decode_ref(q, k, v, [L], 0.5, window=w)
    seen = np.nonzero(o[0, 0])[0]
    assert list(seen) == list(range(L - w, L))


def test_window_paged_and_fp8_forms():
    from oracle.fp8 import dequantize_ref, gqa_decode_fp8_ref
    q, k, v = rand(2, 4, 16), rand(2, 40, 2, 16), rand(2, 40, 2, 16)
    lens, w, ps = [40, 23], 9, 16
    want = gqa_decode_ref(q, k, v, lens, 0.2, window=w)
    # pages in reverse order; entries of blocks before the window are -1
    table = np.array([[-1, 1, 0], [-1, 3, -1]])
    pool_k, pool_v = np.zeros((4, ps, 2, 16)), np.zeros((4, ps, 2, 16))
    for b, L in enumerate(lens):
        for t in range(max(0, L - w), L):
            pool_k[table[b, t // ps], t % ps] = k[b, t]
            pool_v[table[b, t // ps], t % ps] = v[b, t]
    got = OA.gqa_decode_paged_ref(q, pool_k, pool_v, table, ps, lens, 0.2, window=w)
    np.testing.assert_allclose(got[0], want[0], atol=1e-13)
    codes = RNG.integers(0, 126, size=(2, 40, 2, 16)).astype(np.uint8)
    sc = RNG.uniform(0.5, 2.0, size=(2, 40, 2))
    got8 = gqa_decode_fp8_ref(q, codes, codes, sc, sc, lens, 0.2, window=w)
    dq = dequantize_ref(codes, sc)
    want8 = gqa_decode_ref(q, dq, dq, lens, 0.2, window=w)
    np.testing.assert_allclose(got8[0], want8[0], atol=1e-13)


def test_planted_off_by_one_window_fails_the_row_count_pin(monkeypatch):
    orig = OA.gqa_decode_ref

    def off_by_one(q, k, v, seq_lens, scale, window=0):
        # [L - w, L] read as w + 1 rows
        return orig(q, k, v, seq_lens, scale, window + 1 if window > 0 else 0)
    monkeypatch.setattr(OA, "gqa_decode_ref", off_by_one)
    global gqa_decode_ref
    saved = gqa_decode_ref
    gqa_decode_ref = off_by_one
    try:
        with pytest.raises(AssertionError):
            test_window_sees_at_most_w_rows()
    finally:
        gqa_decode_ref = saved


# ----------------------------------------------------------------------------
# E4M3 encoder and the fp8 append oracle
# ----------------------------------------------------------------------------

def test_e4m3_encoder_inverts_the_decoder_and_rounds_to_even():
    from oracle.fp8 import e4m3_encode, e4m3_to_float
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # finite codes
    vals = e4m3_to_float(codes)
    got = e4m3_encode(vals.astype(np.float32))
    # +0 and -0 both encode by their sign; every other value round-trips
    assert np.array_equal(got, codes)
    # midpoints between neighbours go to the even mantissa
    pos = np.sort(e4m3_to_float(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2
    enc = e4m3_encode(mids.astype(np.float32))
    dec = e4m3_to_float(enc)
    lo_code = e4m3_encode(pos[:-1].astype(np.float32))
    hi_code = e4m3_encode(pos[1:].astype(np.float32))
    even = np.where(lo_code % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(dec, even), "ties must go to the even code"
    assert np.all((enc == lo_code) | (enc == hi_code))
    # clamping: beyond 448 the largest finite code, never NaN
    assert list(e4m3_encode(np.array([448.0, 460.0, 1e6, -1e30], np.float32))) == [0x7E, 0x7E, 0x7E, 0xFE]


def test_e4m3_encoder_agrees_with_torch():
    from oracle.fp8 import e4m3_encode
    x = (RNG.standard_normal(20000) * np.exp2(RNG.uniform(-12, 8, 20000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), want)


def test_fp8_append_oracle_scales_and_codes():
    from oracle.fp8 import dequantize_ref, gqa_append_rope_fp8_ref
    from oracle.rope import STYLE_HALF
    q, k, v = rand(3, 8, 64), rand(3, 2, 64), rand(3, 2, 64)
    v[1, 1] = 0.0                                        # an all-zero row: scale 0, codes 0
    out = gqa_append_rope_fp8_ref(q, k, v, [5, -1, 7], 10, 64, STYLE_HALF)
    q_rot, k_rot, kc, ks, vc, vs, written = out
    assert list(written) == [True, False, True]
    np.testing.assert_allclose(ks, np.abs(k_rot).max(-1) / 448, rtol=1e-7)
    assert vs[1, 1] == 0 and not vc[1, 1].any()
    # each row's largest magnitude maps to 448, and decoding is within half a step
    for codes, sc, x in ((kc, ks, k_rot), (vc, vs, v)):
        dq = dequantize_ref(codes, sc)
        rel = np.abs(dq - x) / np.maximum(np.abs(x).max(-1, keepdims=True), 1e-30)
        assert rel.max() <= 2.0 ** -4 + 1e-6
    # static scales are used as given
    st = (np.full((3, 2), 0.01), np.full((3, 2), 0.02))
    _, _, kc2, ks2, _, vs2, _ = gqa_append_rope_fp8_ref(q, k, v, [5, 0, 7], 10, 64, STYLE_HALF, static_scales=st)
    assert np.all(ks2 == np.float32(0.01)) and np.all(vs2 == np.float32(0.02))


def test_fp8_paged_oracle_equals_the_contiguous_one():
    from oracle.fp8 import gqa_decode_fp8_paged_ref, gqa_decode_fp8_ref
    B, L, Hkv, D, ps = 2, 70, 2, 16, 32
    q = rand(B, 4, D)
    codes_k = RNG.integers(0, 126, size=(B, L, Hkv, D)).astype(np.uint8)
    codes_v = RNG.integers(0, 126, size=(B, L, Hkv, D)).astype(np.uint8)
    sk, sv = RNG.uniform(0.5, 2, (B, L, Hkv)), RNG.uniform(0.5, 2, (B, L, Hkv))
    lens = [70, 40]
    table = np.array([[4, 0, 2], [-1, 3, -1]])         # sequence 1 only attends its window
    pk = np.full((5, ps, Hkv, D), 0x7F, np.uint8)
    pv = pk.copy()
    psk, psv = np.full((5, ps, Hkv), np.nan), np.full((5, ps, Hkv), np.nan)
    for b, Lb in enumerate(lens):
        for t in range(Lb):
            page = table[b, t // ps]
            if page < 0:
                continue
            pk[page, t % ps], pv[page, t % ps] = codes_k[b, t], codes_v[b, t]
            psk[page, t % ps], psv[page, t % ps] = sk[b, t], sv[b, t]
    w = 8                                                 # rows 32..39 of sequence 1 lie on page 3
    for win in (0, w):
        lens_used = lens if win == 0 else lens
        want = gqa_decode_fp8_ref(q, codes_k, codes_v, sk, sv, lens_used, 0.3, window=win)
        if win == 0:   # sequence 1's first block is released: compare sequence 0 only
            got = gqa_decode_fp8_paged_ref(q[:1], pk, pv, psk, psv, table[:1], ps, lens[:1], 0.3)
            np.testing.assert_allclose(got[0], want[0][:1], atol=1e-13)
        else:
            got = gqa_decode_fp8_paged_ref(q, pk, pv, psk, psv, table, ps, lens, 0.3, window=win)
            np.testing.assert_allclose(got[0], want[0], atol=1e-13)
            np.testing.assert_allclose(got[1], want[1], atol=1e-13)
