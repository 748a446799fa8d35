"""GPU parity of the cache append with rotary position embedding (the step
before decode: "KV Cache 如何影响了 LLM Inference", section 2.2; "Attention
variants and KV cache", sections 4.2 and 4.4) against the fp64 oracle
(oracle/rope.py), through the C ABI via the Python binding.

Bar, per element: copied entries (values, latents, entries past the rotary
dim) bit-exact; rotated entries within 2^-8 |ref| (one bf16 rounding; 2^-22
for fp32 rows) + 2^-20 (|a| + |b|) for the float32 products of the pair
(a, b). Every cache row other than the appended one must be unchanged, and
skipped sequences must leave everything as it was.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_bf16_amd as da
import workloads as W
from gpu_util import announce, bf16_tensor, f32_tensor
from oracle.attention import gqa_decode_ref
from oracle.rope import (STYLE_HALF, STYLE_INTERLEAVED, apply_rope_ref, gqa_append_rope_ref,
                         mla_append_rope_ref, rope_pairs)

pytestmark = pytest.mark.gpu

STYLES = {"half": STYLE_HALF, "interleaved": STYLE_INTERLEAVED}


def to_dev(a, dtype):
    return bf16_tensor(a) if dtype == "bf16" else f32_tensor(a)


def host_f64(t):
    if t.dtype == torch.bfloat16:
        return W.bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def as_bf16(x):
    """float64 values as stored in bf16 (round to nearest even)."""
    return W.bf16_to_f32(W.bf16_round(np.asarray(x, np.float32))).astype(np.float64)


def rope_bound(x, ref, r, style, dtype):
    """Per-element bound for rotated x (float64 [..., n]) against ref."""
    a, b = rope_pairs(r, style)
    pair_mag = np.zeros_like(x)
    m = np.abs(x[..., a]) + np.abs(x[..., b])
    pair_mag[..., a] = m
    pair_mag[..., b] = m
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -22
    return rel * np.abs(ref) + 2.0 ** -20 * pair_mag


def assert_rotated(got, x, ref, r, style, dtype, what):
    bound = rope_bound(x, ref, r, style, dtype)
    err = np.abs(got - ref)
    bad = err[..., :r] > bound[..., :r]
    assert not bad.any(), f"{what}: {bad.sum()} rotated entries off (max err {err[..., :r].max():.3e})"
    assert np.array_equal(got[..., r:], ref[..., r:]), f"{what}: entries past the rotary dim changed"


def gqa_case(B, Hq, Hkv, D, L, dtype="bf16", r=None, style="half", positions=None, seed=1,
             inv_freq=None, in_place=False, paged=0, base=10000.0, one_page_each=False):
    announce(f"gqa append B{B} Hq{Hq} Hkv{Hkv} D{D} L{L} {dtype} r{r} {style} paged{paged} "
             f"in_place{in_place} pos{None if positions is None else list(positions)[:4]}")
    r = D if r is None else r
    inp = W.make_gqa_append(B, Hq, Hkv, D, L, dtype=dtype, seed=seed, positions=positions)
    q, kn, vn = (to_dev(x, dtype) for x in (inp.q, inp.k_new, inp.v_new))
    pos = torch.from_numpy(inp.positions).cuda()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    table = None
    if paged:
        if one_page_each:
            # every block of sequence b maps to page b: a small pool serves
            # any position
            tab, npages = np.repeat(np.arange(B, dtype=np.int32)[:, None], -(-L // paged), 1), B
        else:
            tab, npages = W.make_block_table([L] * B, paged, seed=seed)
        shape = (npages, paged, Hkv, D)
        table = torch.from_numpy(np.ascontiguousarray(tab, np.int32)).cuda()
    else:
        shape = (B, L, Hkv, D)
    fill = torch.full(shape, 1.0, dtype=tdt, device="cuda")
    kc, vc = fill.clone(), fill.clone()
    k0, v0 = kc.clone(), vc.clone()
    inv = None if inv_freq is None else torch.from_numpy(inv_freq.astype(np.float32)).cuda()
    q_keep = q.clone()
    q_out = da.gqa_append_rope(q, kn, vn, pos, kc, vc, rotary_dim=r, style=style, inv_freq=inv,
                               q_out=q if in_place else None, block_table=table,
                               page_size=paged, max_seq_len=L if paged else None, base=base)
    torch.cuda.synchronize()
    qf, knf, vnf = inp.f64("q"), inp.f64("k_new"), inp.f64("v_new")
    tab_np = None if table is None else table.cpu().numpy()
    written = (inp.positions >= 0) & (inp.positions < L)
    rows = [(b, (b, int(p)) if table is None else (int(tab_np[b, p // paged]), int(p) % paged))
            for b, p in enumerate(inp.positions) if written[b]]
    if fill.numel() <= 2 ** 22:
        # small caches: the whole oracle append, compared entry by entry
        q_ref, k_ref, v_ref, w_ref = gqa_append_rope_ref(
            qf, knf, vnf, inp.positions, host_f64(k0), host_f64(v0), L, r, STYLES[style], base=base,
            inv_freq=inv_freq, block_table=tab_np, page_size=paged)
        assert np.array_equal(w_ref, written)
        got_k, got_v = host_f64(kc), host_f64(vc)
        assert np.array_equal(got_v, v_ref), "v cache: appended rows must be exact copies, others unchanged"
        mask = np.zeros(got_k.shape[:2], bool)
        for b, (i, t) in rows:
            mask[i, t] = True
            assert_rotated(got_k[i, t], knf[b], k_ref[i, t], r, STYLES[style], dtype, f"k row {b}")
        assert np.array_equal(got_k[~mask], k_ref[~mask]), "k cache rows other than the appended ones changed"
    else:
        # full-size caches: the oracle's rotation for the appended rows, and
        # on the GPU every other row compared with its copy taken before
        q_ref = apply_rope_ref(qf, np.where(written, inp.positions, 0), r, STYLES[style], base, inv_freq)
        k_rot = apply_rope_ref(knf, np.where(written, inp.positions, 0), r, STYLES[style], base, inv_freq)
        ek, ev = k0.clone(), v0.clone()
        for b, (i, t) in rows:
            assert_rotated(host_f64(kc[i, t]), knf[b], k_rot[b], r, STYLES[style], dtype, f"k row {b}")
            assert np.array_equal(host_f64(vc[i, t]), vnf[b]), f"v row {b} must be an exact copy"
            ek[i, t] = kc[i, t]
            ev[i, t] = vc[i, t]
        assert torch.equal(kc, ek) and torch.equal(vc, ev), "rows other than the appended ones changed"
    got_q = host_f64(q_out)
    if written.any():
        assert_rotated(got_q[written], qf[written], q_ref[written], r, STYLES[style], dtype, "q")
    if in_place:   # skipped sequences leave their queries as they were
        assert np.array_equal(got_q[~written], host_f64(q_keep)[~written]), "skipped q rows changed in place"
    return inp, q_out, kc, vc


def test_config2_shape():
    gqa_case(32, 32, 8, 128, 4096)


@pytest.mark.parametrize("style", ["half", "interleaved"])
@pytest.mark.parametrize("D,r", [(128, 128), (128, 64), (64, 64), (64, 8)])
def test_styles_and_partial_rotation(style, D, r):
    gqa_case(5, 8, 2, D, 300, r=r, style=style, seed=4)


def test_fp32_cache():
    gqa_case(3, 4, 2, 64, 50, dtype="f32", seed=5)


def test_skipped_and_edge_positions():
    # -1 and L_max skip; 0 and L_max - 1 are the first and last rows
    gqa_case(4, 8, 8, 128, 64, positions=[-1, 0, 63, 64], seed=6, in_place=True)


def test_in_place_mqa_large_positions():
    # angles up to 3e5 rad for the fastest pair
    gqa_case(3, 32, 1, 128, 300000, positions=[299999, 131071, 7], seed=7, in_place=True,
             paged=16, one_page_each=True)


def test_given_frequencies():
    inv = (10000.0 ** (-np.arange(32) / 32.0)) / 8.0          # a stretched base
    gqa_case(3, 8, 2, 64, 500, inv_freq=inv, style="interleaved", seed=8)


def test_paged_pools():
    gqa_case(6, 16, 4, 128, 96, paged=16, seed=9)
    gqa_case(2, 8, 2, 64, 4096, paged=256, style="interleaved", seed=10, base=500000.0)


def test_strided_new_rows_from_one_projection():
    # q, k_new, v_new as views into one [B, (Hq + 2 Hkv) * D] projection output
    announce("gqa append, k/v views of a fused projection")
    B, Hq, Hkv, D, L = 4, 8, 2, 128, 200
    inp = W.make_gqa_append(B, Hq, Hkv, D, L, seed=11)
    qkv = torch.cat([bf16_tensor(inp.q).reshape(B, -1), bf16_tensor(inp.k_new).reshape(B, -1),
                     bf16_tensor(inp.v_new).reshape(B, -1)], dim=1)
    q = qkv[:, :Hq * D].view(B, Hq, D)
    kn = qkv[:, Hq * D:(Hq + Hkv) * D].view(B, Hkv, D)
    vn = qkv[:, (Hq + Hkv) * D:].view(B, Hkv, D)
    assert kn.stride() == ((Hq + 2 * Hkv) * D, D, 1)
    pos = torch.from_numpy(inp.positions).cuda()
    kc = torch.zeros((B, L, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    q_out = da.gqa_append_rope(q, kn, vn, pos, kc, vc)
    kc2, vc2 = torch.zeros_like(kc), torch.zeros_like(kc)
    q_out2 = da.gqa_append_rope(bf16_tensor(inp.q), bf16_tensor(inp.k_new), bf16_tensor(inp.v_new),
                                pos, kc2, vc2)
    torch.cuda.synchronize()
    assert torch.equal(q_out.view(torch.int16), q_out2.view(torch.int16))
    assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))


def test_append_then_decode_matches_the_oracle_pipeline():
    announce("gqa append then decode")
    B, Hq, Hkv, D, L = 3, 16, 4, 128, 700
    cache = W.make_gqa(B, Hq, Hkv, D, [L] * B, seed=12)
    lens = np.array([700, 1, 345], np.int32)
    app = W.make_gqa_append(B, Hq, Hkv, D, L, seed=13, positions=lens - 1)
    kc, vc = bf16_tensor(cache.k), bf16_tensor(cache.v)
    q_rot = da.gqa_append_rope(bf16_tensor(app.q), bf16_tensor(app.k_new), bf16_tensor(app.v_new),
                               torch.from_numpy(app.positions).cuda(), kc, vc)
    sl = torch.from_numpy(lens).cuda()
    out, lse = da.gqa_decode(q_rot, kc, vc, sl)
    torch.cuda.synchronize()
    q_ref, k_ref, v_ref, _ = gqa_append_rope_ref(app.f64("q"), app.f64("k_new"), app.f64("v_new"),
                                                 app.positions, cache.as_f64("k"), cache.as_f64("v"),
                                                 L, D, STYLE_HALF)
    # the rotated rows are stored in the cache's type (bf16) before decode reads them
    ro, rl = gqa_decode_ref(as_bf16(q_ref), as_bf16(k_ref), v_ref, lens, 1 / np.sqrt(D))
    err = np.abs(out.cpu().numpy() - ro).max(axis=-1) / np.abs(ro).max(axis=-1)
    assert err.max() <= 1e-2 and np.abs(lse.cpu().numpy() - rl).max() <= 1e-3


# ----------------------------------------------------------------------------
# MLA
# ----------------------------------------------------------------------------

def mla_case(B, H, L, style="half", positions=None, seed=1, paged=0, in_place=False, r=64):
    announce(f"mla append B{B} H{H} L{L} {style} r{r} paged{paged} in_place{in_place}")
    inp = W.make_mla_append(B, H, L, seed=seed, positions=positions)
    qr, kvn = bf16_tensor(inp.q), bf16_tensor(inp.k_new)
    pos = torch.from_numpy(inp.positions).cuda()
    table = None
    if paged:
        tab, npages = W.make_block_table([L] * B, paged, seed=seed)
        table = torch.from_numpy(np.ascontiguousarray(tab, np.int32)).cuda()
        shape = (npages, paged, 576)
    else:
        shape = (B, L, 576)
    cache = torch.full(shape, 1.0, dtype=torch.bfloat16, device="cuda")
    c0 = cache.clone()
    q_keep = qr.clone()
    q_out = da.mla_append_rope(qr, kvn, pos, cache, rotary_dim=r, style=style,
                               q_rope_out=qr if in_place else None, block_table=table,
                               page_size=paged, max_seq_len=L if paged else None)
    torch.cuda.synchronize()
    tab_np = None if table is None else table.cpu().numpy()
    written = (inp.positions >= 0) & (inp.positions < L)
    kvf, qf = inp.f64("k_new"), inp.f64("q")
    rows = [(b, (b, int(p)) if table is None else (int(tab_np[b, p // paged]), int(p) % paged))
            for b, p in enumerate(inp.positions) if written[b]]
    if cache.numel() <= 2 ** 22:
        q_ref, c_ref, w_ref = mla_append_rope_ref(qf, kvf, inp.positions, host_f64(c0), L, r,
                                                  STYLES[style], block_table=tab_np, page_size=paged)
        assert np.array_equal(w_ref, written)
        got_c = host_f64(cache)
        mask = np.zeros(got_c.shape[:2], bool)
        for b, (i, t) in rows:
            mask[i, t] = True
            assert np.array_equal(got_c[i, t, :512], kvf[b, :512]), "latent must be copied exactly"
            assert_rotated(got_c[i, t, 512:], kvf[b, 512:], c_ref[i, t, 512:], r, STYLES[style], "bf16",
                           "k_rope")
        assert np.array_equal(got_c[~mask], c_ref[~mask]), "cache rows other than the appended ones changed"
    else:
        pos0 = np.where(written, inp.positions, 0)
        q_ref = apply_rope_ref(qf, pos0, r, STYLES[style])
        k_rot = apply_rope_ref(kvf[:, 512:], pos0, r, STYLES[style])
        expect = c0.clone()
        for b, (i, t) in rows:
            row = host_f64(cache[i, t])
            assert np.array_equal(row[:512], kvf[b, :512]), "latent must be copied exactly"
            assert_rotated(row[512:], kvf[b, 512:], k_rot[b], r, STYLES[style], "bf16", "k_rope")
            expect[i, t] = cache[i, t]
        assert torch.equal(cache, expect), "cache rows other than the appended ones changed"
    got_q = host_f64(q_out)
    assert_rotated(got_q[written], qf[written], q_ref[written], r, STYLES[style], "bf16", "q_rope")
    if in_place:
        assert np.array_equal(got_q[~written], host_f64(q_keep)[~written])


def test_mla_config3_shape():
    mla_case(64, 128, 4096)


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_mla_styles_and_heads(style):
    mla_case(5, 16, 100, style=style, seed=3)
    mla_case(3, 96, 33, style=style, seed=4, r=32)


def test_mla_skipped_in_place_and_paged():
    mla_case(4, 32, 64, positions=[63, -5, 64, 0], seed=5, in_place=True)
    mla_case(6, 128, 256, paged=64, seed=6)


def test_mla_append_then_decode_uses_the_rotated_rows():
    announce("mla append then decode")
    B, H, L = 2, 16, 300
    base = W.make_mla(B, H, [L] * B, seed=21)
    lens = np.array([300, 17], np.int32)
    app = W.make_mla_append(B, H, L, seed=22, positions=lens - 1)
    cache = bf16_tensor(base.cache)
    q_rot = da.mla_append_rope(bf16_tensor(app.q), bf16_tensor(app.k_new),
                               torch.from_numpy(app.positions).cuda(), cache)
    out, lse = da.mla_decode_absorbed(bf16_tensor(base.q_nope), q_rot, cache, bf16_tensor(base.w_uk),
                                      bf16_tensor(base.w_uv), torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    from oracle.attention import mla_absorbed_ref
    q_ref, c_ref, _ = mla_append_rope_ref(app.f64("q"), app.f64("k_new"), app.positions,
                                          W.bf16_to_f32(base.cache).astype(np.float64), L, 64, STYLE_HALF)
    ro, rl = mla_absorbed_ref(W.bf16_to_f32(base.q_nope).astype(np.float64), as_bf16(q_ref), as_bf16(c_ref), lens,
                              W.bf16_to_f32(base.w_uk).astype(np.float64),
                              W.bf16_to_f32(base.w_uv).astype(np.float64), 1 / np.sqrt(192))
    err = np.abs(out.cpu().numpy() - ro).max(axis=-1) / np.abs(ro).max(axis=-1)
    assert err.max() <= 1e-2 and np.abs(lse.cpu().numpy() - rl).max() <= 1e-3


def test_error_codes_with_real_buffers():
    announce("append error codes")
    q = torch.zeros((2, 8, 64), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((2, 2, 64), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((2, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    for kw in ({"rotary_dim": 12}, {"rotary_dim": 72}, {"base": 1.0}, {"base": float("inf")}):
        with pytest.raises(da.DecodeAttnError):
            da.gqa_append_rope(q, kn, kn, pos, kc, kc.clone(), **kw)
    with pytest.raises(ValueError):
        da.gqa_append_rope(q, kn, kn, pos, kc, kc.clone(), style="diagonal")
    with pytest.raises(ValueError):
        da.gqa_append_rope(q, kn, kn, pos.long(), kc, kc.clone())


# ----------------------------------------------------------------------------
# E4M3 caches
# ----------------------------------------------------------------------------

def e4m3_step(y):
    """Spacing of E4M3 values around |y|."""
    a = np.abs(y)
    return np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))


@pytest.mark.parametrize("static", [False, True])
@pytest.mark.parametrize("style,r", [("half", None), ("interleaved", 64)])
def test_fp8_append(static, style, r):
    from oracle.fp8 import e4m3_to_float, gqa_append_rope_fp8_ref
    B, Hq, Hkv, D, L = 6, 16, 4, 128, 300
    announce(f"gqa append fp8 static{static} {style} r{r}")
    inp = W.make_gqa_append(B, Hq, Hkv, D, L, seed=41, positions=[0, 299, -1, 150, 300, 7])
    rr = D if r is None else r
    q, kn, vn = (bf16_tensor(x) for x in (inp.q, inp.k_new, inp.v_new))
    pos = torch.from_numpy(inp.positions).cuda()
    kc = torch.full((B, L, Hkv, D), 0x11, dtype=torch.uint8, device="cuda")
    vc = kc.clone()
    k0 = kc.clone()
    if static:
        sk = np.array([0.01, 0.02, 0.005, 0.03], np.float32)
        sv = np.array([0.02, 0.01, 0.04, 0.008], np.float32)
        ks = torch.from_numpy(sk).cuda().expand(B, L, Hkv)
        vs = torch.from_numpy(sv).cuda().expand(B, L, Hkv)
        static_np = (np.broadcast_to(sk, (B, Hkv)), np.broadcast_to(sv, (B, Hkv)))
    else:
        ks = torch.full((B, L, Hkv), -1.0, device="cuda")
        vs = ks.clone()
        static_np = None
    ks0, vs0 = ks.clone(), vs.clone()
    q_out = da.gqa_append_rope_fp8(q, kn, vn, pos, kc, vc, ks, vs, rotary_dim=rr, style=style)
    torch.cuda.synchronize()
    qf, knf, vnf = inp.f64("q"), inp.f64("k_new"), inp.f64("v_new")
    q_rot, k_rot, kcode, ksc, vcode, vsc, written = gqa_append_rope_fp8_ref(
        qf, knf, vnf, inp.positions, L, rr, STYLES[style], static_scales=static_np)
    assert_rotated(host_f64(q_out)[written], qf[written], q_rot[written], rr, STYLES[style], "bf16", "q")
    kc_h, vc_h = kc.cpu().numpy(), vc.cpu().numpy()
    ks_h, vs_h = ks.cpu().numpy(), vs.cpu().numpy()
    mask = np.zeros((B, L), bool)
    for b in np.nonzero(written)[0]:
        p = int(inp.positions[b])
        mask[b, p] = True
        # values: the same float32 decision on both sides, so codes and scales are equal
        assert np.array_equal(vc_h[b, p], vcode[b]), f"v codes of row {b}"
        assert np.array_equal(vs_h[b, p], vsc[b]), f"v scales of row {b}"
        # keys: rotated in float32 by the kernel, in float64 by the oracle; the
        # scale agrees to float32 rounding and each code is a nearest E4M3 value
        np.testing.assert_allclose(ks_h[b, p], ksc[b], rtol=2.0 ** -20)
        y = np.clip(k_rot[b] / ksc[b][:, None].astype(np.float64), -448.0, 448.0)   # clamped codes
        dec = e4m3_to_float(kc_h[b, p])
        assert np.all(np.abs(dec - y) <= 0.5 * e4m3_step(y) * (1 + 1e-3) + 1e-6 * np.abs(y)), f"k codes of row {b}"
    others = ~mask
    assert np.array_equal(kc_h[others], k0.cpu().numpy()[others]) and np.array_equal(vc_h[others], k0.cpu().numpy()[others])
    if not static:
        assert np.array_equal(ks_h[others], ks0.cpu().numpy()[others])
        assert np.array_equal(vs_h[others], vs0.cpu().numpy()[others])


def test_fp8_append_then_decode():
    from oracle.fp8 import dequantize_ref
    announce("gqa append fp8 then decode")
    B, Hq, Hkv, D, L = 3, 32, 8, 128, 500
    cache = W.make_gqa_fp8(B, Hq, Hkv, D, [L] * B, seed=42, pad_nan=False)
    lens = np.array([500, 1, 257], np.int32)
    app = W.make_gqa_append(B, Hq, Hkv, D, L, seed=43, positions=lens - 1)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kc, vc, ks, vs = d(cache.k), d(cache.v), d(cache.k_scale), d(cache.v_scale)
    q_rot = da.gqa_append_rope_fp8(bf16_tensor(app.q), bf16_tensor(app.k_new), bf16_tensor(app.v_new),
                                   d(app.positions), kc, vc, ks, vs)
    out, lse = da.gqa_decode_fp8(q_rot, kc, vc, ks, vs, d(lens), 1 / np.sqrt(D))
    torch.cuda.synchronize()
    # the oracle decodes the cache the kernel left (codes and scales as written)
    kd = dequantize_ref(kc.cpu().numpy(), ks.cpu().numpy())
    vd = dequantize_ref(vc.cpu().numpy(), vs.cpu().numpy())
    ro, rl = gqa_decode_ref(host_f64(q_rot), kd, vd, lens, 1 / np.sqrt(D))
    err = np.abs(out.cpu().numpy() - ro).max(axis=-1) / np.abs(ro).max(axis=-1)
    assert err.max() <= 1e-2 and np.abs(lse.cpu().numpy() - rl).max() <= 1e-3


def test_recorded_call_replays_the_same_launch():
    # the binding's recorded_calls(): repeating the recorded C call does what
    # the wrapper call did (the bench's append steps rely on it)
    announce("recorded call replay")
    B, Hq, Hkv, D, L = 4, 8, 2, 128, 64
    inp = W.make_gqa_append(B, Hq, Hkv, D, L, seed=61)
    q, kn, vn = (bf16_tensor(x) for x in (inp.q, inp.k_new, inp.v_new))
    pos = torch.from_numpy(inp.positions).cuda()
    kc = torch.zeros((B, L, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vc, qo = torch.zeros_like(kc), torch.empty_like(q)
    with da.recorded_calls() as rec:
        da.gqa_append_rope(q, kn, vn, pos, kc, vc, q_out=qo)
    torch.cuda.synchronize()
    (fn, args), = rec
    want = (kc.clone(), vc.clone(), qo.clone())
    kc.zero_(); vc.zero_(); qo.zero_()
    assert fn(*args) == 0
    torch.cuda.synchronize()
    for got, w in zip((kc, vc, qo), want):
        assert torch.equal(got.view(torch.int16), w.view(torch.int16))
