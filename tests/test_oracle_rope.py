"""Pin the fp64 rotary-embedding and cache-append oracle (oracle/rope.py) to
things other than itself.

  * the rotation as complex multiplication, (a + ib) e^{i m theta}: an
    independent formulation that fixes the direction and the pairing;
  * the pages' identity R_m^T R_n = R_{n-m} ("Attention variants and KV
    cache", section 4.4): rotated dot products depend only on n - m;
  * closed forms: position 0 is the identity, the fastest pair turns by m
    radians, r = 4 at base 10^4 has frequencies 1 and 1/100, norms are kept;
  * the two pairings are the same rotation under a permutation of entries;
  * caller-given frequencies; composition R_m R_n = R_{m+n};
  * append: only row m changes, v and c_kv are copied exactly, skipped
    sequences change nothing, paged rows land where the table says;
  * end to end: decode attention over a cache built by appends is unchanged
    when every position is shifted by the same amount.
The planted-mistake tests at the end check that pins fail on broken copies.
"""
import math

import numpy as np
import pytest

import oracle.rope as R
from oracle.attention import gqa_decode_ref, mla_absorbed_ref

RNG = np.random.default_rng(77)


def rand(*shape):
    return RNG.standard_normal(shape)


def complex_rope(x, m, r, style, base=10000.0):
    """Rotation of one vector x [n] as complex products, built entry by entry."""
    out = [complex(v) for v in x]
    h = r // 2
    res = list(x)
    for i in range(h):
        theta = base ** (-2.0 * i / r)
        ia, ib = (i, i + h) if style == R.STYLE_HALF else (2 * i, 2 * i + 1)
        z = complex(out[ia].real, out[ib].real) * complex(math.cos(m * theta), math.sin(m * theta))
        res[ia], res[ib] = z.real, z.imag
    return np.array(res)


@pytest.mark.parametrize("style", [R.STYLE_HALF, R.STYLE_INTERLEAVED])
@pytest.mark.parametrize("r,n", [(8, 8), (64, 64), (64, 128), (128, 128)])
def test_complex_multiplication_form(style, r, n):
    x = rand(3, 2, n)
    pos = [0, 5, 4093]
    got = R.apply_rope_ref(x, pos, r, style)
    for b, m in enumerate(pos):
        for h in range(2):
            np.testing.assert_allclose(got[b, h], complex_rope(x[b, h], m, r, style), rtol=0, atol=1e-10)


@pytest.mark.parametrize("style", [R.STYLE_HALF, R.STYLE_INTERLEAVED])
def test_relative_position_identity(style):
    # <R_m q, R_n k> = <q, R_{n-m} k> = <R_{m+c} q, R_{n+c} k>
    r = 64
    q, k = rand(1, 1, r), rand(1, 1, r)
    for m, n, c in [(3, 10, 100), (4000, 17, 12345), (0, 0, 7)]:
        lhs = np.dot(R.apply_rope_ref(q, [m], r, style).ravel(), R.apply_rope_ref(k, [n], r, style).ravel())
        mid = np.dot(q.ravel(), R.apply_rope_ref(k, [n - m], r, style).ravel())
        rhs = np.dot(R.apply_rope_ref(q, [m + c], r, style).ravel(),
                     R.apply_rope_ref(k, [n + c], r, style).ravel())
        assert abs(lhs - mid) < 1e-9 and abs(lhs - rhs) < 1e-9


def test_closed_forms():
    # r = 4, base 1e4: theta = (1, 1/100). Interleaved x = e0 + e3 at m = 1:
    # pair 0 (1, 0) turns by 1 rad, pair 1 (0, 1) by 0.01 rad.
    x = np.array([[[1.0, 0.0, 0.0, 1.0]]])
    got = R.apply_rope_ref(x, [1], 4, R.STYLE_INTERLEAVED, base=1e4).ravel()
    want = [math.cos(1), math.sin(1), -math.sin(0.01), math.cos(0.01)]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
    # half pairing of the same frequencies: pairs (0, 2) and (1, 3)
    got = R.apply_rope_ref(x, [1], 4, R.STYLE_HALF, base=1e4).ravel()
    want = [1 * math.cos(1) - 0, 0 * math.cos(0.01) - 1 * math.sin(0.01), math.sin(1), math.cos(0.01)]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
    np.testing.assert_allclose(R.rope_inv_freq(4, 1e4), [1.0, 0.01], rtol=1e-15)
    np.testing.assert_allclose(R.rope_inv_freq(128, 5e5)[64 - 1], 5e5 ** (-126 / 128), rtol=1e-14)


def test_identity_norm_tail():
    x = rand(4, 3, 128)
    np.testing.assert_array_equal(R.apply_rope_ref(x, [0, 0, 0, 0], 128, R.STYLE_HALF), x)
    y = R.apply_rope_ref(x, [1, 99, 4095, 70000], 64, R.STYLE_HALF)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(y[..., 64:], x[..., 64:])      # past r: untouched


def test_pairings_are_one_rotation_permuted():
    # interleaved layout p(x) puts entry i at 2i and entry i + r/2 at 2i + 1
    r = 64
    x = rand(2, 5, r)
    perm = np.empty(r, np.int64)
    perm[0::2] = np.arange(r // 2)
    perm[1::2] = np.arange(r // 2) + r // 2
    half = R.apply_rope_ref(x, [9, 1234], r, R.STYLE_HALF)
    inter = R.apply_rope_ref(x[..., perm], [9, 1234], r, R.STYLE_INTERLEAVED)
    np.testing.assert_allclose(inter, half[..., perm], rtol=0, atol=1e-12)


def test_given_frequencies_and_composition():
    r = 32
    x = rand(1, 2, r)
    theta = R.rope_inv_freq(r, 10000.0)
    # halved frequencies at position 2m == base frequencies at m
    a = R.apply_rope_ref(x, [2 * 37], r, R.STYLE_HALF, inv_freq=theta / 2)
    b = R.apply_rope_ref(x, [37], r, R.STYLE_HALF)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # R_m R_n = R_{m+n}
    c = R.apply_rope_ref(R.apply_rope_ref(x, [300], r, R.STYLE_INTERLEAVED), [45], r, R.STYLE_INTERLEAVED)
    d = R.apply_rope_ref(x, [345], r, R.STYLE_INTERLEAVED)
    np.testing.assert_allclose(c, d, rtol=0, atol=1e-12)


def test_gqa_append_rows():
    B, Hq, Hkv, D, L = 3, 8, 2, 64, 10
    q, kn, vn = rand(B, Hq, D), rand(B, Hkv, D), rand(B, Hkv, D)
    kc, vc = rand(B, L, Hkv, D), rand(B, L, Hkv, D)
    pos = np.array([4, -1, 9])
    qo, k2, v2, w = R.gqa_append_rope_ref(q, kn, vn, pos, kc, vc, L, D, R.STYLE_HALF)
    assert list(w) == [True, False, True]
    for b in range(B):
        for t in range(L):
            if w[b] and t == pos[b]:
                np.testing.assert_array_equal(v2[b, t], vn[b])
                for h in range(Hkv):
                    np.testing.assert_allclose(k2[b, t, h], complex_rope(kn[b, h], t, D, R.STYLE_HALF), atol=1e-12)
            else:
                np.testing.assert_array_equal(k2[b, t], kc[b, t])
                np.testing.assert_array_equal(v2[b, t], vc[b, t])
    assert np.isnan(qo[1]).all()
    for h in range(Hq):
        np.testing.assert_allclose(qo[2, h], complex_rope(q[2, h], 9, D, R.STYLE_HALF), atol=1e-12)
    # a position at max_seq_len is skipped too
    _, k3, _, w3 = R.gqa_append_rope_ref(q, kn, vn, np.array([L, 0, 0]), kc, vc, L, D, R.STYLE_HALF)
    assert not w3[0] and np.array_equal(k3[0], kc[0])


def test_paged_append_lands_on_the_table_page():
    B, Hkv, D, ps, pages = 2, 2, 64, 16, 8
    table = np.array([[5, 2, 7], [1, 0, 3]])
    pool_k, pool_v = rand(pages, ps, Hkv, D), rand(pages, ps, Hkv, D)
    q, kn, vn = rand(B, 4, D), rand(B, Hkv, D), rand(B, Hkv, D)
    pos = np.array([17, 40])                 # block 1 row 1 -> page 2; block 2 row 8 -> page 3
    _, k2, v2, _ = R.gqa_append_rope_ref(q, kn, vn, pos, pool_k, pool_v, 48, 32, R.STYLE_INTERLEAVED,
                                         block_table=table, page_size=ps)
    changed = np.argwhere(np.any(v2 != pool_v, axis=(2, 3)))
    assert sorted(map(tuple, changed)) == [(2, 1), (3, 8)]
    np.testing.assert_array_equal(v2[2, 1], vn[0])
    np.testing.assert_allclose(k2[3, 8, 1], complex_rope(kn[1, 1], 40, 32, R.STYLE_INTERLEAVED), atol=1e-12)
    np.testing.assert_array_equal(k2[3, 8, 1, 32:], kn[1, 1, 32:])


def test_mla_append_row():
    B, H, L = 2, 4, 6
    qr, kvn, cache = rand(B, H, 64), rand(B, 576), rand(B, L, 576)
    pos = np.array([5, 0])
    qo, c2, w = R.mla_append_rope_ref(qr, kvn, pos, cache, L, 64, R.STYLE_INTERLEAVED)
    for b in range(B):
        np.testing.assert_array_equal(c2[b, pos[b], :512], kvn[b, :512])
        np.testing.assert_allclose(c2[b, pos[b], 512:], complex_rope(kvn[b, 512:], pos[b], 64, R.STYLE_INTERLEAVED),
                                   atol=1e-12)
        others = [t for t in range(L) if t != pos[b]]
        np.testing.assert_array_equal(c2[b, others], cache[b, others])
    np.testing.assert_array_equal(qo[1], qr[1])      # position 0: identity


def test_decode_after_appends_depends_on_relative_positions():
    # Fill a cache by appending tokens 0..L-1 at positions c..c+L-1 and query at
    # the last one: GQA and absorbed-MLA results do not depend on c.
    B, Hq, Hkv, D, L = 1, 4, 2, 64, 9
    qs, ks, vs = rand(L, Hq, D), rand(L, Hkv, D), rand(L, Hkv, D)
    outs = []
    for c in (0, 1000):
        kc, vc = np.zeros((B, L, Hkv, D)), np.zeros((B, L, Hkv, D))
        for t in range(L):
            # row t of the cache holds token t, rotated by position c + t
            k_rot = R.apply_rope_ref(ks[t][None], [c + t], D, R.STYLE_HALF)
            kc[0, t] = k_rot[0]
            vc[0, t] = vs[t]
        q_rot = R.apply_rope_ref(qs[-1][None], [c + L - 1], D, R.STYLE_HALF)
        outs.append(gqa_decode_ref(q_rot, kc, vc, [L], 1 / 8))
    np.testing.assert_allclose(outs[0][0], outs[1][0], atol=1e-12)
    np.testing.assert_allclose(outs[0][1], outs[1][1], atol=1e-12)
    # MLA: the cache row is [c_kv ; RoPE(k_rope)] through the append oracle
    H = 2
    w_uk, w_uv = rand(H, 512, 128) * 0.05, rand(H, 512, 128) * 0.05
    qn, qr, kv = rand(1, H, 128), rand(1, H, 64), rand(L, 576)
    res = []
    for c in (3, 777):
        cache = np.zeros((1, L, 576))
        for t in range(L):
            _, cache, _ = R.mla_append_rope_ref(qr, kv[t][None], [t], cache, L, 64, R.STYLE_HALF)
            # the oracle rotated by t; re-rotate the rope part by the shift c
            cache[0, t, 512:] = R.apply_rope_ref(cache[:1, t, 512:], [c], 64, R.STYLE_HALF)[0]
        q_rot = R.apply_rope_ref(qr, [c + L - 1], 64, R.STYLE_HALF)
        res.append(mla_absorbed_ref(qn, q_rot, cache, [L], w_uk, w_uv, 1 / math.sqrt(192)))
    np.testing.assert_allclose(res[0][0], res[1][0], atol=1e-10)


# ----------------------------------------------------------------------------
# planted mistakes: a broken copy of the rotation must fail a pin
# ----------------------------------------------------------------------------

def broken_rope(kind):
    def f(x, positions, r, style, base=10000.0, inv_freq=None):
        x = np.array(x, dtype=np.float64, copy=True)
        theta = R.rope_inv_freq(r, base)
        if kind == "exponent":
            theta = np.power(base, -np.arange(r // 2) / r)          # 2i/r dropped to i/r
        a_idx, b_idx = R.rope_pairs(r, style)
        for bi in range(x.shape[0]):
            phi = positions[bi] * theta
            c, s = np.cos(phi), np.sin(phi)
            a, b = x[bi][..., a_idx].copy(), x[bi][..., b_idx].copy()
            if kind == "sign":
                x[bi][..., a_idx], x[bi][..., b_idx] = a * c + b * s, -a * s + b * c
            else:
                x[bi][..., a_idx], x[bi][..., b_idx] = a * c - b * s, a * s + b * c
        return x
    return f


@pytest.mark.parametrize("kind", ["sign", "exponent"])
def test_planted_mistakes_fail_the_complex_pin(kind, monkeypatch):
    monkeypatch.setattr(R, "apply_rope_ref", broken_rope(kind))
    with pytest.raises(AssertionError):
        test_complex_multiplication_form(R.STYLE_HALF, 64, 64)
