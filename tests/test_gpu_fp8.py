"""GPU parity of GQA decode over an FP8 (E4M3) cache ("Attention variants and
KV cache", arganzheng.life, section 6.3) against the fp64 oracle, through
the C ABI via the Python binding.

The kernel decodes every code exactly (E4M3 values are bf16 values); its
roundings are fp32 sums, the per-row scale products and (on the matrix cores)
the softmax weights rounded to bf16 for the value product. Besides the bar,
each row is held to the error that weight rounding can cause, computed from
the data (gpu_util.bf16_weight_bound). Rows past each length
hold the NaN code and NaN scales, so any read past the end poisons the row.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_bf16_amd as da
import workloads as W
from gpu_util import announce, assert_parity, bf16_tensor, bf16_weight_bound
from oracle.fp8 import dequantize_ref, gqa_decode_fp8_ref

pytestmark = pytest.mark.gpu


def to_device(inp):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return (bf16_tensor(inp.q), dev(inp.k), dev(inp.v), dev(inp.k_scale), dev(inp.v_scale),
            dev(inp.seq_lens.astype(np.int32)))


def run(inp, num_splits=0, scales=None):
    q, k, v, ks, vs, sl = to_device(inp)
    if scales is not None:
        ks, vs = scales
    out, lse = da.gqa_decode_fp8(q, k, v, ks, vs, sl, inp.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def oracle_rows(inp, seqs):
    """The oracle one sequence per call (bounded memory at full size)."""
    outs, lses = [], []
    for b in seqs:
        L = int(max(1, inp.seq_lens[b]))
        q = W.bf16_to_f32(inp.q[b:b + 1]).astype(np.float64)
        o, l = gqa_decode_fp8_ref(q, inp.k[b:b + 1, :L], inp.v[b:b + 1, :L], inp.k_scale[b:b + 1, :L],
                                  inp.v_scale[b:b + 1, :L], inp.seq_lens[b:b + 1], inp.scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


def check(inp, out, lse, seqs=None, what=""):
    seqs = list(range(len(inp.seq_lens)) if seqs is None else seqs)
    ro, rl = oracle_rows(inp, seqs)
    assert_parity(out[seqs], lse[seqs], ro, rl, what=what)
    Lm = int(max(1, inp.seq_lens[seqs].max()))
    kv = [dequantize_ref(x[seqs, :Lm], s[seqs, :Lm]) for x, s in ((inp.k, inp.k_scale), (inp.v, inp.v_scale))]
    kv = [np.nan_to_num(x) for x in kv]                      # padded rows are never attended
    q = W.bf16_to_f32(inp.q[seqs]).astype(np.float64)
    bound = bf16_weight_bound(q, kv[0], kv[1], inp.seq_lens[seqs], inp.scale, ro, rl)
    assert_parity(out[seqs], lse[seqs], ro, rl, out_rtol=bound, lse_atol=1e-4, what=what + " tight")


def test_config2_shapes_reduced_batch_all_rows():
    announce("gqa fp8 B4 Hq32 Hkv8 D128 L4096")
    inp = W.make_gqa_fp8(4, 32, 8, 128, [4096, 4096, 4096, 4096], seed=3)
    out, lse = run(inp)
    check(inp, out, lse, what="fp8 B4")


def test_config2_full_size_all_rows():
    announce("gqa fp8 config2 full B32 L4096, every row")
    inp = W.make_gqa_fp8_config(2)
    out, lse = run(inp)
    ro, rl = oracle_rows(inp, range(32))
    assert_parity(out, lse, ro, rl, what="fp8 config2")


EDGE = [
    # B, Hq, Hkv, D, lens
    (4, 8, 2, 128, [0, 1, 15, 17]),                    # empty, L = 1, ragged tails
    (2, 32, 1, 128, [700, 2049]),                      # MQA, g = 32
    (3, 12, 4, 128, [100, 64, 1]),                     # g = 3 (no reduce-scatter path)
    (2, 8, 8, 128, [3000, 5000]),                      # MHA: few units, 16-wave workgroups
    (2, 16, 2, 64, [129, 4000]),                       # D = 64
    (3, 14, 2, 64, [33, 1, 517]),                      # D = 64, g = 7
    (16, 32, 8, 128, [4096, 1, 0, 2000, 129, 4095, 77, 3000,
                      1024, 33, 2500, 4096, 0, 640, 1500, 2]),   # 8-wave, 2 splits
    (64, 32, 32, 128, [(i % 5) * 97 + (i % 3) for i in range(64)]),   # longest-first order
]


@pytest.mark.parametrize("B,Hq,Hkv,D,lens", EDGE)
def test_edge_cases(B, Hq, Hkv, D, lens):
    announce(f"gqa fp8 edge B{B} Hq{Hq} Hkv{Hkv} D{D} lens{lens}")
    inp = W.make_gqa_fp8(B, Hq, Hkv, D, lens, seed=13, max_seq_len=max(lens) + 5)
    out, lse = run(inp)
    check(inp, out, lse, what="fp8 edge")


@pytest.mark.parametrize("splits", [1, 3, 16])
def test_split_count_invariance(splits):
    announce(f"gqa fp8 splits S={splits}")
    inp = W.make_gqa_fp8(3, 16, 4, 128, [2500, 1, 777], seed=6, max_seq_len=2600)
    out, lse = run(inp, num_splits=splits)
    check(inp, out, lse, what=f"fp8 S={splits}")


def test_per_head_scales_through_zero_strides():
    # one scale per KV head: a [Hkv] vector expanded to [B, L, Hkv] with zero
    # batch and token strides gives the same result as the full array
    announce("gqa fp8 per-head scales (broadcast strides)")
    inp = W.make_gqa_fp8(3, 16, 4, 128, [1000, 333, 2048], seed=8, max_seq_len=2048, scales="head",
                         pad_nan=False)
    ks_h = torch.from_numpy(inp.k_scale[0, 0].copy()).cuda()
    vs_h = torch.from_numpy(inp.v_scale[0, 0].copy()).cuda()
    B, L, H = inp.k_scale.shape
    ks_b, vs_b = ks_h.expand(B, L, H), vs_h.expand(B, L, H)
    assert ks_b.stride() == (0, 0, 1)
    out_b, lse_b = run(inp, scales=(ks_b, vs_b))
    out_f, lse_f = run(inp)
    assert np.array_equal(out_b, out_f) and np.array_equal(lse_b, lse_f)
    check(inp, out_b, lse_b, what="per-head scales")


def test_fp8_matches_the_bf16_kernel_on_exact_values():
    # scales that are powers of two make every dequantized element an exact
    # bf16 value: the bf16 path on those values must give the same result to
    # fp32 rounding
    announce("gqa fp8 vs bf16 kernel on exact values")
    inp = W.make_gqa_fp8(2, 32, 8, 128, [1500, 4096], seed=2, max_seq_len=4096, pad_nan=False)
    inp.k_scale[:] = np.float32(2.0 ** -6)
    inp.v_scale[:] = np.float32(2.0 ** -5)
    out8, lse8 = run(inp)
    kb = W.bf16_round(dequantize_ref(inp.k, inp.k_scale).astype(np.float32))
    vb = W.bf16_round(dequantize_ref(inp.v, inp.v_scale).astype(np.float32))
    sl = torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda()
    out16, lse16 = da.gqa_decode(bf16_tensor(inp.q), bf16_tensor(kb), bf16_tensor(vb), sl, inp.scale)
    np.testing.assert_allclose(out8, out16.cpu().numpy(), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(lse8, lse16.cpu().numpy(), rtol=0, atol=1e-5)


def test_error_codes_with_real_buffers():
    announce("gqa fp8 error codes")
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 16, 2, 128), dtype=torch.uint8, device="cuda")
    s = torch.ones((2, 16, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        da.gqa_decode_fp8(q.float(), k, k, s, s)               # q must be bf16
    with pytest.raises(ValueError):
        da.gqa_decode_fp8(q, k, k, s[:, :8], s)                 # scale shape
    out, lse = da.gqa_decode_fp8(q, k, k, s, s)                 # all-zero codes: mean of zeros
    assert torch.all(out == 0) and torch.allclose(lse, torch.full_like(lse, float(np.log(16))))


# ----------------------------------------------------------------------------
# paged E4M3 pools ("Attention variants and KV cache", sections 6.1 and 6.3)
# ----------------------------------------------------------------------------

def paged_fp8(inp, ps, seed, window=0):
    """Codes and scales paged through one table (seeded random page order);
    unused pool rows hold the NaN code and NaN scales, and with a window the
    pages wholly before the window's first 32-row step are released (entry
    -1, contents NaN)."""
    lens = inp.seq_lens
    table, n_pages = W.make_block_table(lens, ps, seed=seed)
    kp = W.paginate(inp.k, lens, table, n_pages, ps, W.FP8_NAN_CODE)
    vp = W.paginate(inp.v, lens, table, n_pages, ps, W.FP8_NAN_CODE)
    ksp = W.paginate(inp.k_scale, lens, table, n_pages, ps, np.float32("nan"))
    vsp = W.paginate(inp.v_scale, lens, table, n_pages, ps, np.float32("nan"))
    if window:
        for b, L in enumerate(lens):
            first = (max(0, int(L) - window) & ~31) // ps
            for j in range(first):
                for arr, fill in ((kp, W.FP8_NAN_CODE), (vp, W.FP8_NAN_CODE), (ksp, np.nan), (vsp, np.nan)):
                    arr[table[b, j]] = fill
                table[b, j] = -1
    return kp, vp, ksp, vsp, table


@pytest.mark.parametrize("B,Hq,Hkv,lens,ps,window,splits", [
    (4, 32, 8, [4096, 700, 33, 0], 32, 0, 0),
    (3, 16, 2, [3000, 17, 2049], 64, 0, 0),
    (3, 16, 2, [3000, 17, 2049], 256, 1000, 0),
    (2, 8, 8, [5000, 3333], 32, 0, 0),                 # MHA, few units
    (3, 16, 4, [2500, 1, 777], 32, 300, 5),
])
def test_paged_fp8(B, Hq, Hkv, lens, ps, window, splits):
    from oracle.fp8 import gqa_decode_fp8_paged_ref
    announce(f"gqa fp8 paged B{B} Hq{Hq} Hkv{Hkv} ps{ps} w{window} S{splits} lens{lens}")
    inp = W.make_gqa_fp8(B, Hq, Hkv, 128, lens, seed=51)
    kp, vp, ksp, vsp, table = paged_fp8(inp, ps, seed=52, window=window)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out, lse = da.gqa_decode_fp8_paged(bf16_tensor(inp.q), d(kp), d(vp), d(ksp), d(vsp), d(table), ps,
                                       d(inp.seq_lens.astype(np.int32)), max_seq_len=inp.k.shape[1],
                                       softmax_scale=inp.scale, num_splits=splits, window=window)
    torch.cuda.synchronize()
    q64 = W.bf16_to_f32(inp.q).astype(np.float64)
    ro, rl = gqa_decode_fp8_paged_ref(q64, kp, vp, ksp, vsp, table, ps, inp.seq_lens, inp.scale, window=window)
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, what="fp8 paged")


def test_paged_fp8_config2_full_size_all_rows():
    from oracle.fp8 import gqa_decode_fp8_paged_ref
    announce("gqa fp8 paged config2 full B32 L4096 ps32, every row")
    inp = W.make_gqa_fp8_config(2)
    kp, vp, ksp, vsp, table = paged_fp8(inp, 32, seed=53)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out, lse = da.gqa_decode_fp8_paged(bf16_tensor(inp.q), d(kp), d(vp), d(ksp), d(vsp), d(table), 32,
                                       d(inp.seq_lens.astype(np.int32)), softmax_scale=inp.scale)
    torch.cuda.synchronize()
    ro, rl = [], []
    for b in range(32):   # one sequence per oracle call, on its own pages (renumbered)
        pages = table[b, :-(-int(inp.seq_lens[b]) // 32)]
        tab = np.arange(len(pages), dtype=np.int32)[None]
        q64 = W.bf16_to_f32(inp.q[b:b + 1]).astype(np.float64)
        o, l = gqa_decode_fp8_paged_ref(q64, kp[pages], vp[pages], ksp[pages], vsp[pages], tab, 32,
                                        inp.seq_lens[b:b + 1], inp.scale)
        ro.append(o[0])
        rl.append(l[0])
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), np.stack(ro), np.stack(rl), what="fp8 paged config2")


def test_paged_fp8_per_head_scales():
    from oracle.fp8 import gqa_decode_fp8_paged_ref
    announce("gqa fp8 paged per-head scales")
    inp = W.make_gqa_fp8(3, 16, 4, 128, [1000, 333, 2048], seed=54, max_seq_len=2048, scales="head",
                         pad_nan=False)
    kp, vp, _, _, table = paged_fp8(inp, 64, seed=55)
    kh, vh = inp.k_scale[0, 0].copy(), inp.v_scale[0, 0].copy()
    n_pages = kp.shape[0]
    ks = torch.from_numpy(kh).cuda().expand(n_pages, 64, 4)
    vs = torch.from_numpy(vh).cuda().expand(n_pages, 64, 4)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out, lse = da.gqa_decode_fp8_paged(bf16_tensor(inp.q), d(kp), d(vp), ks, vs, d(table), 64,
                                       d(inp.seq_lens.astype(np.int32)), max_seq_len=2048,
                                       softmax_scale=inp.scale)
    torch.cuda.synchronize()
    q64 = W.bf16_to_f32(inp.q).astype(np.float64)
    ksp = np.broadcast_to(kh, (n_pages, 64, 4))
    vsp = np.broadcast_to(vh, (n_pages, 64, 4))
    ro, rl = gqa_decode_fp8_paged_ref(q64, kp, vp, ksp, vsp, table, 64, inp.seq_lens, inp.scale)
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, what="fp8 paged per-head scales")


# ----------------------------------------------------------------------------
# head-major code storage: [B, Hkv, L, D] (or [pages, Hkv, page_size, D]),
# given to the library as a strided [B, L, Hkv, D] view; scales token-major
# ----------------------------------------------------------------------------

def head_major(x):
    """Codes [X, T, H, D] stored head-major on the GPU, returned as the
    [X, T, H, D] view of that storage (strides (H T D, D, T D, 1))."""
    t = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).cuda()
    return t.permute(0, 2, 1, 3)


def test_head_major_codes_config2_full_size_all_rows():
    announce("gqa fp8 config2 full B32 L4096, head-major codes, every row")
    inp = W.make_gqa_fp8_config(2)
    q, k, v, ks, vs, sl = to_device(inp)
    kh, vh = head_major(inp.k), head_major(inp.v)
    assert kh.stride() == (8 * inp.k.shape[1] * 128, 128, inp.k.shape[1] * 128, 1)
    out, lse = da.gqa_decode_fp8(q, kh, vh, ks, vs, sl, inp.scale)
    out_t, lse_t = da.gqa_decode_fp8(q, k, v, ks, vs, sl, inp.scale)
    torch.cuda.synchronize()
    # the same values through other addresses: the same arithmetic, bit for bit
    assert torch.equal(out, out_t) and torch.equal(lse, lse_t)
    ro, rl = oracle_rows(inp, range(32))
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, what="fp8 config2 head-major")


@pytest.mark.parametrize("B,Hq,Hkv,lens,ps,window,splits", [
    (4, 32, 8, [4096, 700, 33, 0], 32, 0, 0),
    (3, 16, 2, [3000, 17, 2049], 64, 1000, 0),
    (3, 16, 4, [2500, 1, 777], 32, 0, 5),
])
def test_paged_head_major_pages(B, Hq, Hkv, lens, ps, window, splits):
    from oracle.fp8 import gqa_decode_fp8_paged_ref
    announce(f"gqa fp8 paged head-major pages B{B} Hq{Hq} Hkv{Hkv} ps{ps} w{window} S{splits} lens{lens}")
    inp = W.make_gqa_fp8(B, Hq, Hkv, 128, lens, seed=57)
    kp, vp, ksp, vsp, table = paged_fp8(inp, ps, seed=58, window=window)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    args = (d(ksp), d(vsp), d(table), ps, d(inp.seq_lens.astype(np.int32)))
    kw = dict(max_seq_len=inp.k.shape[1], softmax_scale=inp.scale, num_splits=splits, window=window)
    out, lse = da.gqa_decode_fp8_paged(bf16_tensor(inp.q), head_major(kp), head_major(vp), *args, **kw)
    out_t, lse_t = da.gqa_decode_fp8_paged(bf16_tensor(inp.q), d(kp), d(vp), *args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, out_t) and torch.equal(lse, lse_t)
    q64 = W.bf16_to_f32(inp.q).astype(np.float64)
    ro, rl = gqa_decode_fp8_paged_ref(q64, kp, vp, ksp, vsp, table, ps, inp.seq_lens, inp.scale, window=window)
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, what="fp8 paged head-major")


def test_paged_head_major_pages_config2_full_size_all_rows():
    from oracle.fp8 import gqa_decode_fp8_paged_ref
    announce("gqa fp8 paged config2 full B32 L4096 ps32, head-major pages, every row")
    inp = W.make_gqa_fp8_config(2)
    kp, vp, ksp, vsp, table = paged_fp8(inp, 32, seed=53)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out, lse = da.gqa_decode_fp8_paged(bf16_tensor(inp.q), head_major(kp), head_major(vp), d(ksp), d(vsp),
                                       d(table), 32, d(inp.seq_lens.astype(np.int32)), softmax_scale=inp.scale)
    torch.cuda.synchronize()
    ro, rl = [], []
    for b in range(32):   # one sequence per oracle call, on its own pages (renumbered)
        pages = table[b, :-(-int(inp.seq_lens[b]) // 32)]
        tab = np.arange(len(pages), dtype=np.int32)[None]
        q64 = W.bf16_to_f32(inp.q[b:b + 1]).astype(np.float64)
        o, l = gqa_decode_fp8_paged_ref(q64, kp[pages], vp[pages], ksp[pages], vsp[pages], tab, 32,
                                        inp.seq_lens[b:b + 1], inp.scale)
        ro.append(o[0])
        rl.append(l[0])
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), np.stack(ro), np.stack(rl),
                  what="fp8 paged config2 head-major")
