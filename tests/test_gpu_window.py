"""GPU parity of sliding-window GQA decode ("Attention variants and KV
cache", section 5.3: each query sees only the latest w keys) against the fp64
oracle, through the C ABI via the Python binding.

Rows outside the window are poisoned: on contiguous caches the rows before
L - w hold NaN (they must not be read); on paged pools the table entries of
blocks before the window's first page are -1 and those pages hold NaN (the
rows of the window's first page before L - w are read with weight 0, so they
keep their finite values). Rows past each length hold NaN as in the other
tests. Besides the 1e-2 bar every row is held to the error that rounding the
softmax weights to bf16 can cause (the matrix-core kernel), computed from the
window's rows.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_bf16_amd as da
import workloads as W
from gpu_util import announce, assert_parity, bf16_tensor, bf16_weight_bound, f32_tensor
from oracle.attention import gqa_decode_ref
from oracle.fp8 import dequantize_ref, gqa_decode_fp8_ref

pytestmark = pytest.mark.gpu


def f64(a, dtype):
    return W.bf16_to_f32(a).astype(np.float64) if dtype == "bf16" else a.astype(np.float64)


def dev(a, dtype):
    return bf16_tensor(a) if dtype == "bf16" else f32_tensor(a)


def nan_of(dtype):
    return W.BF16_NAN_BITS if dtype == "bf16" else np.float32("nan")


def window_rows(k, v, lens, w):
    """The window's rows of each sequence moved to the front: full attention
    over them equals the windowed attention (pinned in the oracle tests)."""
    B = k.shape[0]
    Lw = max(1, min(int(max(lens)), w))
    ks = np.zeros((B, Lw) + k.shape[2:])
    vs = np.zeros((B, Lw) + v.shape[2:])
    lw = np.zeros(B, np.int64)
    for b, L in enumerate(lens):
        lo = max(0, int(L) - w)
        n = int(L) - lo
        ks[b, :n], vs[b, :n], lw[b] = k[b, lo:L], v[b, lo:L], n
    return ks, vs, lw


def check(q, k, v, lens, scale, w, out, lse, what):
    ro, rl = gqa_decode_ref(q, k, v, lens, scale, window=w)
    assert_parity(out, lse, ro, rl, what=what)
    ks, vs, lw = window_rows(k, v, lens, w)
    bound = bf16_weight_bound(q, ks, vs, lw, scale, ro, rl)
    assert_parity(out, lse, ro, rl, out_rtol=bound, lse_atol=1e-4, what=what + " tight")


def poison_before_window(cache, lens, w, dtype):
    c = cache.copy()
    for b, L in enumerate(lens):
        c[b, :max(0, int(L) - w)] = nan_of(dtype)
    return c


CASES = [
    # B, Hq, Hkv, D, lens, w, dtype, splits
    (32, 32, 8, 128, [4096] * 32, 1000, "bf16", 0),           # Llama-3-8B GQA shape, one split
    (4, 32, 8, 128, [4096, 700, 1, 0], 1024, "bf16", 0),       # few units: split windows
    (3, 16, 2, 128, [3000, 17, 2049], 100, "bf16", 0),
    (3, 16, 2, 128, [3000, 17, 2049], 1, "bf16", 0),          # only the newest row
    (2, 8, 8, 128, [5000, 3333], 777, "bf16", 0),              # MHA, few units (16-wave plan)
    (3, 8, 2, 64, [500, 64, 129], 50, "f32", 0),               # fp32: vector-ALU kernel
    (3, 16, 4, 128, [2500, 1, 777], 300, "bf16", 3),           # forced splits
    (3, 16, 4, 128, [2500, 1, 777], 300, "bf16", 16),
    (2, 32, 4, 128, [1000, 200], 5000, "bf16", 0),             # a window longer than the cache
]


@pytest.mark.parametrize("B,Hq,Hkv,D,lens,w,dtype,splits", CASES)
def test_contiguous(B, Hq, Hkv, D, lens, w, dtype, splits):
    announce(f"gqa window B{B} Hq{Hq} Hkv{Hkv} D{D} w{w} {dtype} S{splits} lens{lens[:4]}")
    inp = W.make_gqa(B, Hq, Hkv, D, lens, dtype=dtype, seed=31, pad_value=float("nan"))
    k = poison_before_window(inp.k, lens, w, dtype)
    v = poison_before_window(inp.v, lens, w, dtype)
    sl = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    out, lse = da.gqa_decode(dev(inp.q, dtype), dev(k, dtype), dev(v, dtype), sl, inp.scale,
                             num_splits=splits, window=w)
    torch.cuda.synchronize()
    seqs = list(range(B)) if B <= 8 else [0, 13, 31]
    q64, k64, v64 = (f64(x, dtype)[seqs] for x in (inp.q, inp.k, inp.v))
    check(q64, np.nan_to_num(k64), np.nan_to_num(v64), np.asarray(lens)[seqs], inp.scale, w,
          out.cpu().numpy()[seqs], lse.cpu().numpy()[seqs], f"window {w}")


@pytest.mark.parametrize("ps,w,splits", [(16, 100, 0), (16, 37, 0), (64, 1000, 0), (16, 300, 5)])
def test_paged(ps, w, splits):
    announce(f"gqa window paged ps{ps} w{w} S{splits}")
    lens = [3000, 17, 2049, 333]
    B, Hq, Hkv, D = 4, 16, 4, 128
    inp = W.make_gqa(B, Hq, Hkv, D, lens, seed=32, pad_value=float("nan"))
    table, n_pages = W.make_block_table(lens, ps, seed=33)
    fill = W.BF16_NAN_BITS
    kp = W.paginate(inp.k, lens, table, n_pages, ps, fill)
    vp = W.paginate(inp.v, lens, table, n_pages, ps, fill)
    for b, L in enumerate(lens):                  # blocks wholly before the window: released
        first = (max(0, L - w) & ~15) // ps
        for j in range(first):
            kp[table[b, j]] = fill
            vp[table[b, j]] = fill
            table[b, j] = -1
    sl = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    out, lse = da.gqa_decode_paged(bf16_tensor(inp.q), bf16_tensor(kp), bf16_tensor(vp),
                                   torch.from_numpy(table).cuda(), ps, sl, max_seq_len=inp.k.shape[1],
                                   softmax_scale=inp.scale, num_splits=splits, window=w)
    torch.cuda.synchronize()
    check(f64(inp.q, "bf16"), np.nan_to_num(f64(inp.k, "bf16")), np.nan_to_num(f64(inp.v, "bf16")),
          lens, inp.scale, w, out.cpu().numpy(), lse.cpu().numpy(), f"paged window {w}")


@pytest.mark.parametrize("B,Hq,Hkv,lens,w", [
    (4, 32, 8, [4096, 700, 1, 0], 1024),          # matrix-core fp8 path
    (2, 8, 8, [3000, 5000], 500),                 # MHA, few units: vector-ALU fp8 path
])
def test_fp8(B, Hq, Hkv, lens, w):
    announce(f"gqa window fp8 B{B} Hq{Hq} Hkv{Hkv} w{w}")
    inp = W.make_gqa_fp8(B, Hq, Hkv, 128, lens, seed=34)
    k, v = inp.k.copy(), inp.v.copy()
    ks, vs = inp.k_scale.copy(), inp.v_scale.copy()
    for b, L in enumerate(lens):
        lo = max(0, L - w)
        k[b, :lo] = W.FP8_NAN_CODE
        v[b, :lo] = W.FP8_NAN_CODE
        ks[b, :lo] = np.nan
        vs[b, :lo] = np.nan
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out, lse = da.gqa_decode_fp8(bf16_tensor(inp.q), d(k), d(v), d(ks), d(vs),
                                 torch.from_numpy(np.asarray(lens, np.int32)).cuda(), inp.scale, window=w)
    torch.cuda.synchronize()
    q64 = W.bf16_to_f32(inp.q).astype(np.float64)
    Lm = max(1, max(lens))
    ro, rl = gqa_decode_fp8_ref(q64, inp.k[:, :Lm], inp.v[:, :Lm], inp.k_scale[:, :Lm], inp.v_scale[:, :Lm],
                                lens, inp.scale, window=w)
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, what="fp8 window")
    kd = np.nan_to_num(dequantize_ref(inp.k[:, :Lm], inp.k_scale[:, :Lm]))
    vd = np.nan_to_num(dequantize_ref(inp.v[:, :Lm], inp.v_scale[:, :Lm]))
    kw, vw, lw = window_rows(kd, vd, lens, w)
    bound = bf16_weight_bound(q64, kw, vw, lw, inp.scale, ro, rl)
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, out_rtol=bound, lse_atol=1e-4,
                  what="fp8 window tight")


def test_window_query_sizes_cover_paged_calls():
    # the split count for a window is planned on w + 15 rows, for paged and
    # contiguous calls alike, and never exceeds the unwindowed plan's
    announce("window split planning")
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 4096, 2, 128), dtype=torch.bfloat16, device="cuda")
    for w in (1, 16, 128, 129, 1000, 4081, 4096, 10000):
        s_w = da.gqa_num_splits(q, k, window=w)
        assert 1 <= s_w <= da.gqa_num_splits(q, k)
    with pytest.raises(da.DecodeAttnError):
        da.gqa_decode(q, k, k, None, window=-1)
