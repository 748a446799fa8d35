"""GPU parity of the paged-cache entry points (block table + shared pool,
"Attention variants and KV cache", arganzheng.life, section 6.1 on paging)
against the fp64 paged oracle, through the C ABI via the Python binding.

Pools are built from the same seeded contiguous caches the other GPU tests
use: each sequence's rows are scattered over pages in a seeded random
physical order (workloads.make_block_table / paginate), and every pool row
that no table entry covers for a valid token (spare pages, the tail of a
last page) holds NaN, so a read of a wrong row poisons the result. Table
entries past a sequence's pages are -1 and must never be read.

Besides the oracle, a paged call is compared with the contiguous call on the
same data: where both plan the same splits, they run the same arithmetic in
the same order and must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_bf16_amd as da
import workloads as W
from gpu_util import (announce, assert_parity, bf16_tensor, bf16_weight_bound, f32_tensor, gqa_to_device,
                      mla_to_device)
from oracle.attention import gqa_decode_paged_ref, mla_absorbed_paged_ref

pytestmark = pytest.mark.gpu

NAN = float("nan")


def _fill(dtype):
    return W.BF16_NAN_BITS if dtype == "bf16" else np.float32("nan")


def _f64(a, dtype):
    return W.bf16_to_f32(a).astype(np.float64) if dtype == "bf16" else a.astype(np.float64)


def _dev(a, dtype):
    return bf16_tensor(a) if dtype == "bf16" else f32_tensor(a)


def gqa_paged_inputs(inp, page_size, seed=5, max_blocks=None, share_prefix=0):
    """(k_pool, v_pool, table) on the host for a GQAInputs. share_prefix > 0
    makes sequence 1 reuse sequence 0's first share_prefix pages (its rows
    there are made equal to sequence 0's first)."""
    lens = inp.seq_lens
    table, n_pages = W.make_block_table(lens, page_size, seed=seed, max_blocks=max_blocks)
    if share_prefix:
        rows = share_prefix * page_size
        assert lens[0] >= rows and lens[1] >= rows
        inp.k[1, :rows] = inp.k[0, :rows]
        inp.v[1, :rows] = inp.v[0, :rows]
        table[1, :share_prefix] = table[0, :share_prefix]
    fill = _fill(inp.dtype)
    kp = W.paginate(inp.k, lens, table, n_pages, page_size, fill)
    vp = W.paginate(inp.v, lens, table, n_pages, page_size, fill)
    return kp, vp, table


def run_gqa_paged(inp, kp, vp, table, page_size, num_splits=0):
    q = _dev(inp.q, inp.dtype)
    sl = torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda()
    out, lse = da.gqa_decode_paged(q, _dev(kp, inp.dtype), _dev(vp, inp.dtype),
                                   torch.from_numpy(table).cuda(), page_size, sl,
                                   max_seq_len=inp.k.shape[1], softmax_scale=inp.scale,
                                   num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def run_gqa_contiguous(inp, num_splits=0):
    q, k, v, sl = gqa_to_device(inp)
    out, lse = da.gqa_decode(q, k, v, sl, inp.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def gqa_bound(inp, ro, rl):
    """Per-row error bound from rounding the weights to bf16 (bf16 caches on
    the matrix cores; gpu_util.bf16_weight_bound), from the contiguous rows."""
    d = inp.dtype
    Lm = int(max(1, inp.seq_lens.max()))
    k = np.nan_to_num(_f64(inp.k[:, :Lm], d))
    v = np.nan_to_num(_f64(inp.v[:, :Lm], d))
    return bf16_weight_bound(_f64(inp.q, d), k, v, inp.seq_lens, inp.scale, ro, rl)


def gqa_oracle(inp, kp, vp, table, page_size, seqs=None):
    """The paged oracle one sequence per call, on that sequence's pages only
    (renumbered), so memory stays bounded at full size."""
    seqs = list(range(len(inp.seq_lens)) if seqs is None else seqs)
    d = inp.dtype
    outs, lses = [], []
    for b in seqs:
        pages = table[b, :max(1, -(-int(inp.seq_lens[b]) // page_size))]
        tab = np.arange(len(pages), dtype=np.int32)[None]
        o, l = gqa_decode_paged_ref(_f64(inp.q[b:b + 1], d), _f64(kp[pages], d), _f64(vp[pages], d), tab,
                                    page_size, inp.seq_lens[b:b + 1], inp.scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


GQA_CASES = [
    # B, Hq, Hkv, D, lens, dtype, page_size, num_splits
    (4, 8, 2, 128, [0, 1, 15, 16], "bf16", 16, 0),
    (5, 32, 8, 128, [17, 1000, 2049, 4096, 333], "bf16", 16, 0),
    (5, 32, 8, 128, [17, 1000, 2049, 4096, 333], "bf16", 64, 3),
    (3, 16, 4, 128, [2500, 1, 777], "bf16", 32, 7),
    (2, 32, 1, 128, [700, 2049], "bf16", 256, 0),          # MQA
    (3, 8, 8, 64, [129, 4000, 31], "bf16", 16, 0),         # MHA, D=64
    (2, 6, 6, 64, [31, 2], "f32", 16, 0),
    (3, 8, 4, 128, [513, 77, 1024], "f32", 128, 2),
    (2, 8, 8, 128, [3000, 5000], "bf16", 16, 0),           # 16-wave workgroups, many splits
]


@pytest.mark.parametrize("B,Hq,Hkv,D,lens,dtype,page_size,splits", GQA_CASES)
def test_gqa_paged_matches_oracle(B, Hq, Hkv, D, lens, dtype, page_size, splits):
    announce(f"gqa paged B{B} Hq{Hq} Hkv{Hkv} D{D} lens{lens} {dtype} page{page_size} S{splits}")
    inp = W.make_gqa(B, Hq, Hkv, D, lens, dtype, seed=31, max_seq_len=max(lens) + 9,
                     pad_value=NAN)
    kp, vp, table = gqa_paged_inputs(inp, page_size, max_blocks=-(-(max(lens) + 9) // page_size))
    out, lse = run_gqa_paged(inp, kp, vp, table, page_size, splits)
    ro, rl = gqa_oracle(inp, kp, vp, table, page_size)
    assert_parity(out, lse, ro, rl, what="gqa paged")
    assert_parity(out, lse, ro, rl, out_rtol=gqa_bound(inp, ro, rl), lse_atol=1e-4, what="gqa paged tight")


@pytest.mark.parametrize("splits", [1, 4])
def test_gqa_paged_equals_contiguous_bitwise(splits):
    # L = 4096 over 1 or 4 splits: chunks of 4096 / 1024 rows, multiples of
    # 16, so the paged and the contiguous call plan the same splits
    announce(f"gqa paged == contiguous S{splits}")
    inp = W.make_gqa(6, 32, 8, 128, [4096, 1, 0, 2047, 3000, 16], "bf16", seed=12,
                     max_seq_len=4096, pad_value=NAN)
    kp, vp, table = gqa_paged_inputs(inp, 16)
    out_p, lse_p = run_gqa_paged(inp, kp, vp, table, 16, splits)
    out_c, lse_c = run_gqa_contiguous(inp, splits)
    assert np.array_equal(out_p, out_c) and np.array_equal(lse_p, lse_c)


def test_gqa_paged_shared_prefix_pages():
    # two sequences whose first 5 blocks are the same physical pages
    announce("gqa paged shared prefix")
    inp = W.make_gqa(3, 16, 4, 128, [200, 170, 90], "bf16", seed=14, max_seq_len=200,
                     pad_value=NAN)
    kp, vp, table = gqa_paged_inputs(inp, 16, share_prefix=5)
    assert table[0, 4] == table[1, 4]
    out, lse = run_gqa_paged(inp, kp, vp, table, 16)
    ro, rl = gqa_oracle(inp, kp, vp, table, 16)
    assert_parity(out, lse, ro, rl, out_rtol=gqa_bound(inp, ro, rl), lse_atol=1e-4, what="shared prefix")
    # and the same as attending the contiguous caches (rows made equal)
    oc, lc = run_gqa_contiguous(inp)
    assert_parity(oc, lc, ro, rl, out_rtol=gqa_bound(inp, ro, rl), lse_atol=1e-4,
                  what="contiguous, same rows")


def test_gqa_paged_config2_full_size():
    # B32 Hq32 Hkv8 D128 L4096 bf16 in 16-row pages: every row against the
    # contiguous call (same plan: bit for bit) and against the oracle
    announce("gqa paged full B32 Hq32 Hkv8 L4096 page16")
    inp = W.make_gqa_config(2)
    kp, vp, table = gqa_paged_inputs(inp, 16, seed=2)
    out_p, lse_p = run_gqa_paged(inp, kp, vp, table, 16)
    out_c, lse_c = run_gqa_contiguous(inp)
    assert np.array_equal(out_p, out_c) and np.array_equal(lse_p, lse_c)
    ro, rl = gqa_oracle(inp, kp, vp, table, 16)
    assert_parity(out_p, lse_p, ro, rl, what="config2 paged")


# ----------------------------------------------------------------------------
# absorbed MLA
# ----------------------------------------------------------------------------

def mla_paged_inputs(inp, page_size, seed=6, max_blocks=None):
    table, n_pages = W.make_block_table(inp.seq_lens, page_size, seed=seed, max_blocks=max_blocks)
    pool = W.paginate(inp.cache, inp.seq_lens, table, n_pages, page_size, W.BF16_NAN_BITS)
    return pool, table


def run_mla_paged(inp, pool, table, page_size, num_splits=0):
    qn, qr, _, wuk, wuv, sl = mla_to_device(inp)
    out, lse = da.mla_decode_absorbed_paged(qn, qr, bf16_tensor(pool),
                                            torch.from_numpy(table).cuda(), page_size, sl,
                                            wuk, wuv, max_seq_len=inp.cache.shape[1],
                                            softmax_scale=inp.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def run_mla_contiguous(inp, num_splits=0):
    qn, qr, cache, wuk, wuv, sl = mla_to_device(inp)
    out, lse = da.mla_decode_absorbed(qn, qr, cache, wuk, wuv, sl, inp.scale,
                                      num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def assert_mla_paged(inp, pool, table, page_size, out, lse, seqs=None, what=""):
    """The bar against the paged oracle, one sequence at a time: each call
    gets only the sequence's own pages (renumbered), so memory stays bounded
    at full size."""
    seqs = list(range(len(inp.seq_lens)) if seqs is None else seqs)
    f = lambda a: W.bf16_to_f32(a).astype(np.float64)
    wuk, wuv = f(inp.w_uk), f(inp.w_uv)
    ro, rl = [], []
    for b in seqs:
        L = int(inp.seq_lens[b])
        pages = table[b, :max(1, -(-L // page_size))]
        tab = np.arange(len(pages), dtype=np.int32)[None]
        o, l = mla_absorbed_paged_ref(f(inp.q_nope[b:b + 1]), f(inp.q_rope[b:b + 1]), f(pool[pages]), tab,
                                      page_size, inp.seq_lens[b:b + 1], wuk, wuv, inp.scale)
        ro.append(o[0])
        rl.append(l[0])
    return assert_parity(out[seqs], lse[seqs], np.stack(ro), np.stack(rl), what=what)


MLA_CASES = [
    # B, H, lens, page_size, num_splits
    (4, 128, [1, 31, 33, 0], 16, 0),
    (5, 128, [2048, 17, 4000, 129, 64], 16, 0),
    (5, 128, [2048, 17, 4000, 129, 64], 64, 3),
    (3, 64, [100, 1000, 47], 32, 0),
    (2, 32, [65, 4097], 16, 5),
    (3, 96, [1500, 2, 260], 256, 0),                 # three-wave shapes
    (3, 16, [300, 1, 4097], 16, 0),
]


@pytest.mark.parametrize("B,H,lens,page_size,splits", MLA_CASES)
def test_mla_paged_matches_oracle(B, H, lens, page_size, splits):
    announce(f"mla paged B{B} H{H} lens{lens} page{page_size} S{splits}")
    inp = W.make_mla(B, H, lens, seed=41, max_seq_len=max(lens) + 3, pad_value=NAN)
    pool, table = mla_paged_inputs(inp, page_size, max_blocks=-(-(max(lens) + 3) // page_size) + 2)
    out, lse = run_mla_paged(inp, pool, table, page_size, splits)
    assert_mla_paged(inp, pool, table, page_size, out, lse, what="mla paged")
    # both split modes round split starts to 32-row tiles: the contiguous
    # call plans the same splits and must agree bit for bit
    out_c, lse_c = run_mla_contiguous(inp, splits)
    assert np.array_equal(out, out_c) and np.array_equal(lse, lse_c)


def test_mla_paged_stages_compose():
    announce("mla paged stages compose")
    inp = W.make_mla(3, 128, [1500, 40, 3000], seed=6, max_seq_len=3000, pad_value=NAN)
    pool, table = mla_paged_inputs(inp, 16)
    qn, qr, _, wuk, wuv, sl = mla_to_device(inp)
    pool_d, table_d = bf16_tensor(pool), torch.from_numpy(table).cuda()
    absorb, attend, merge, out_s, lse_s, _ = da.mla_stages(qn, qr, pool_d, wuk, wuv, sl, inp.scale,
                                                           paged=(table_d, 16, 3000))
    absorb()
    attend()
    merge()
    out, lse = da.mla_decode_absorbed_paged(qn, qr, pool_d, table_d, 16, sl, wuk, wuv,
                                            max_seq_len=3000, softmax_scale=inp.scale)
    assert torch.equal(out, out_s) and torch.equal(lse, lse_s)


def test_mla_paged_config3_full_size():
    # B64 H128 L4096 in 64-row pages: every row against the contiguous call
    # and against the oracle
    announce("mla paged full B64 H128 L4096 page64")
    inp = W.make_mla_config(3)
    pool, table = mla_paged_inputs(inp, 64, seed=3)
    out_p, lse_p = run_mla_paged(inp, pool, table, 64)
    out_c, lse_c = run_mla_contiguous(inp)
    assert np.array_equal(out_p, out_c) and np.array_equal(lse_p, lse_c)
    assert_mla_paged(inp, pool, table, 64, out_p, lse_p, what="config3 paged")


def test_paged_error_codes_with_real_buffers():
    announce("paged error codes")
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((8, 16, 2, 128), dtype=torch.bfloat16, device="cuda")
    sl = torch.tensor([10, 20], dtype=torch.int32, device="cuda")
    table = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(da.DecodeAttnError) as e:      # 2 blocks of 16 < 64 rows
        da.gqa_decode_paged(q, pool, pool, table, 16, sl, max_seq_len=64)
    assert e.value.status == 1
    pool8 = torch.zeros((8, 8, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(da.DecodeAttnError) as e:      # pages of 8 rows
        da.gqa_decode_paged(q, pool8, pool8, torch.zeros((2, 4), dtype=torch.int32, device="cuda"),
                            8, sl)
    assert e.value.status == 1
