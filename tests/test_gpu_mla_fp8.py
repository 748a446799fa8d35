"""GPU parity of absorbed-MLA decode over an E4M3 latent cache (c_kv and
k_rope ranges scaled apart) against the fp64 oracle, called through the C
ABI via the Python binding.

The bar is the bf16 path's: row-relative output error <= 1e-2 and |lse
error| <= 1e-3 on every sequence. The oracle dequantizes each row range by
range (oracle.fp8.dequantize_mla_rows_ref) and attends in fp64; the kernel
keeps the codes exact (E4M3 values are bf16 values) and applies the scales in
fp32, so its only roundings are the bf16 query and weights, as for a bf16
cache.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_bf16_amd as da
import workloads as W
from gpu_util import announce, assert_parity, bf16_tensor, f32_tensor
from oracle.fp8 import mla_absorbed_fp8_ref

pytestmark = pytest.mark.gpu


def f64(bits):
    return W.bf16_to_f32(bits).astype(np.float64)


def oracle_rows(inp, seqs, scale_nope=None, scale_rope=None):
    """The oracle one sequence at a time (bounded memory), stacked."""
    sn = inp.scale_nope if scale_nope is None else scale_nope
    sr = inp.scale_rope if scale_rope is None else scale_rope
    wuk, wuv = f64(inp.w_uk), f64(inp.w_uv)
    outs, lses = [], []
    for b in seqs:
        L = max(int(inp.seq_lens[b]), 1)
        o, l = mla_absorbed_fp8_ref(f64(inp.q_nope[b:b + 1]), f64(inp.q_rope[b:b + 1]),
                                    inp.cache[b:b + 1, :L], sn[b:b + 1, :L], sr[b:b + 1, :L],
                                    inp.seq_lens[b:b + 1], wuk, wuv, inp.scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


def to_device(inp):
    return (bf16_tensor(inp.q_nope), bf16_tensor(inp.q_rope), torch.from_numpy(inp.cache).cuda(),
            f32_tensor(inp.scale_nope), f32_tensor(inp.scale_rope), bf16_tensor(inp.w_uk),
            bf16_tensor(inp.w_uv), torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda())


def run(inp, num_splits=0):
    qn, qr, codes, sn, sr, wuk, wuv, sl = to_device(inp)
    out, lse = da.mla_decode_absorbed_fp8(qn, qr, codes, sn, sr, wuk, wuv, sl, inp.scale,
                                          num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(inp, out, lse, what):
    ro, rl = oracle_rows(inp, range(len(inp.seq_lens)))
    err = assert_parity(out, lse, ro, rl, what=what)
    print(what, "max row rel err, max lse err:", err)
    return err


def test_config3_full_size_all_rows():
    announce("mla fp8 config3 full B64 H128 L4096, every row")
    inp = W.make_mla_fp8_config(3)
    out, lse = run(inp)
    check(inp, out, lse, "mla fp8 config3")


def test_config4_long_context_all_rows():
    announce("mla fp8 config4 B4 H128 L~U[16384,32768] NaN-padded")
    inp = W.make_mla_fp8_config(4)
    out, lse = run(inp)
    check(inp, out, lse, "mla fp8 config4")


EDGE = [
    # B, H, lens
    (4, 128, [1, 2, 31, 33]),
    (3, 128, [0, 32, 0]),            # empty sequences
    (2, 64, [100, 1000]),
    (2, 32, [65, 7]),
    (3, 16, [300, 1, 4097]),         # 16 heads run on a 32-head wave
    (2, 48, [700, 33]),              # 48 on two waves of 32
    (3, 96, [1500, 2, 260]),         # 96 on four waves of 32
    (2, 128, [0, 0]),                # nothing to attend to at all
    (7, 128, [1, 5000, 0, 33, 12000, 64, 2]),
]


@pytest.mark.parametrize("B,H,lens", EDGE)
def test_edge_cases(B, H, lens):
    announce(f"mla fp8 edge B{B} H{H} lens{lens}")
    inp = W.make_mla_fp8(B, H, lens, seed=23, max_seq_len=max(lens) + 5)
    out, lse = run(inp)
    check(inp, out, lse, f"mla fp8 edge {lens}")


@pytest.mark.parametrize("splits", [1, 3, 0, 40])
def test_split_count_invariance(splits):
    announce(f"mla fp8 split invariance S={splits}")
    inp = W.make_mla_fp8(2, 128, [3000, 1200], seed=7, max_seq_len=3001)
    out, lse = run(inp, num_splits=splits)
    check(inp, out, lse, f"mla fp8 S={splits}")
    out2, lse2 = run(inp, num_splits=splits)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_ranges_with_very_different_scales():
    # k_rope drawn 50x larger than c_kv: the two ranges' scales differ by
    # about that factor, which a shared scale would not represent
    announce("mla fp8 rope range 50x the nope range")
    inp = W.make_mla_fp8(3, 128, [2000, 64, 777], seed=9, max_seq_len=2048, rope_std=50.0)
    assert np.nanmedian(inp.scale_rope / inp.scale_nope) > 20
    out, lse = run(inp)
    check(inp, out, lse, "mla fp8 rope x50")


def test_one_scale_per_sequence_through_a_zero_token_stride():
    # scale views [B, L] with stride_t = 0: one (nope, rope) pair per sequence
    announce("mla fp8 per-sequence scales (zero token stride)")
    inp = W.make_mla_fp8(3, 64, [1000, 31, 2100], seed=10, max_seq_len=2100, pad_nan=False)
    B, L = inp.scale_nope.shape
    psn = np.array([0.01, 0.02, 0.005], np.float32)
    psr = np.array([0.3, 0.004, 0.07], np.float32)
    qn, qr, codes, _, _, wuk, wuv, sl = to_device(inp)
    sn = f32_tensor(psn)[:, None].expand(B, L)
    sr = f32_tensor(psr)[:, None].expand(B, L)
    assert sn.stride() == (1, 0)
    out, lse = da.mla_decode_absorbed_fp8(qn, qr, codes, sn, sr, wuk, wuv, sl, inp.scale)
    torch.cuda.synchronize()
    ro, rl = oracle_rows(inp, range(B), np.broadcast_to(psn[:, None], (B, L)),
                         np.broadcast_to(psr[:, None], (B, L)))
    err = assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, what="mla fp8 per-seq scales")
    print("per-sequence scales:", err)


def test_strided_cache_rows():
    # rows 640 bytes apart inside a larger allocation (strides in bytes)
    announce("mla fp8 strided cache rows")
    inp = W.make_mla_fp8(2, 128, [500, 1300], seed=11, max_seq_len=1300)
    qn, qr, codes, sn, sr, wuk, wuv, sl = to_device(inp)
    big = torch.full((2, 1300, 640), 0x7F, dtype=torch.uint8, device="cuda")   # NaN codes around
    big[:, :, :576] = codes
    view = big[:, :, :576]
    assert view.stride() == (1300 * 640, 640, 1)
    out, lse = da.mla_decode_absorbed_fp8(qn, qr, view, sn, sr, wuk, wuv, sl, inp.scale)
    torch.cuda.synchronize()
    ro, rl = oracle_rows(inp, range(2))
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, what="mla fp8 strided")


def test_error_codes_with_real_buffers():
    announce("mla fp8 error codes")
    inp = W.make_mla_fp8(2, 128, [64, 64], seed=12, max_seq_len=64)
    qn, qr, codes, sn, sr, wuk, wuv, sl = to_device(inp)
    with pytest.raises(ValueError):
        da.mla_decode_absorbed_fp8(qn, qr, codes.float(), sn, sr, wuk, wuv, sl)      # codes dtype
    with pytest.raises(ValueError):
        da.mla_decode_absorbed_fp8(qn, qr, codes, sn[:, :8], sr, wuk, wuv, sl)       # scale shape
    with pytest.raises(ValueError):
        da.mla_decode_absorbed_fp8(qn, qr, codes, sn, sr.double(), wuk, wuv, sl)     # scale dtype
    with pytest.raises(da.DecodeAttnError):
        da.mla_decode_absorbed_fp8(qn, qr, codes[:, :, :575], sn, sr, wuk, wuv, sl)  # row width
    # float8_e4m3fn views of the same bytes are accepted
    out, lse = da.mla_decode_absorbed_fp8(qn, qr, codes.view(torch.float8_e4m3fn), sn, sr, wuk, wuv, sl)
    torch.cuda.synchronize()
    ro, rl = oracle_rows(inp, range(2))
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, what="mla fp8 e4m3fn view")


# ----------------------------------------------------------------------------
# paged E4M3 latent pools
# ----------------------------------------------------------------------------

def paged_fp8(inp, ps, seed):
    """Pools of the input's codes and scales in a seeded random page order;
    every pool row that holds no cached row is NaN (code and scales)."""
    table, n_pages = W.make_block_table(inp.seq_lens, ps, seed=seed, spare_pages=3,
                                        max_blocks=-(-inp.cache.shape[1] // ps))
    cp = W.paginate(inp.cache, inp.seq_lens, table, n_pages, ps, W.FP8_NAN_CODE)
    snp = W.paginate(inp.scale_nope, inp.seq_lens, table, n_pages, ps, np.float32(np.nan))
    srp = W.paginate(inp.scale_rope, inp.seq_lens, table, n_pages, ps, np.float32(np.nan))
    return cp, snp, srp, table


def run_paged(inp, ps, seed, num_splits=0):
    from oracle.fp8 import mla_absorbed_fp8_paged_ref
    cp, snp, srp, table = paged_fp8(inp, ps, seed)
    qn, qr = bf16_tensor(inp.q_nope), bf16_tensor(inp.q_rope)
    wuk, wuv = bf16_tensor(inp.w_uk), bf16_tensor(inp.w_uv)
    sl = torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda()
    out, lse = da.mla_decode_absorbed_fp8_paged(qn, qr, torch.from_numpy(cp).cuda(), f32_tensor(snp),
                                                f32_tensor(srp), torch.from_numpy(table).cuda(), ps, sl, wuk,
                                                wuv, max_seq_len=inp.cache.shape[1], softmax_scale=inp.scale,
                                                num_splits=num_splits)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    # the oracle per sequence, through its own pages
    wuk64, wuv64 = f64(inp.w_uk), f64(inp.w_uv)
    ro, rl = [], []
    for b in range(len(inp.seq_lens)):
        o, l = mla_absorbed_fp8_paged_ref(f64(inp.q_nope[b:b + 1]), f64(inp.q_rope[b:b + 1]), cp, snp, srp,
                                          table[b:b + 1], ps, inp.seq_lens[b:b + 1], wuk64, wuv64, inp.scale)
        ro.append(o[0])
        rl.append(l[0])
    return out, lse, np.stack(ro), np.stack(rl)


PAGED = [
    # B, H, lens, page size, splits
    (3, 128, [700, 33, 1], 16, 0),
    (2, 64, [1000, 257], 32, 0),
    (4, 32, [0, 100, 511, 64], 64, 0),
    (2, 16, [300, 2049], 16, 3),
    (3, 96, [1500, 2, 260], 128, 0),
    (2, 48, [129, 700], 16, 0),
]


@pytest.mark.parametrize("B,H,lens,ps,splits", PAGED)
def test_paged_matches_oracle(B, H, lens, ps, splits):
    announce(f"mla fp8 paged B{B} H{H} ps{ps} S{splits} lens{lens}")
    inp = W.make_mla_fp8(B, H, lens, seed=31, max_seq_len=max(lens) + 40)
    out, lse, ro, rl = run_paged(inp, ps, seed=32, num_splits=splits)
    err = assert_parity(out, lse, ro, rl, what=f"mla fp8 paged ps{ps}")
    print("paged errors:", err)


def test_paged_equals_contiguous_bit_for_bit():
    # the same rows, the same split plan: the paged kernel reads the same
    # tiles from other addresses, so the results agree exactly
    announce("mla fp8 paged vs contiguous, bitwise")
    inp = W.make_mla_fp8(4, 128, [2000, 512, 31, 1200], seed=33, max_seq_len=2048)
    out_c, lse_c = run(inp)
    out_p, lse_p, ro, rl = run_paged(inp, 16, seed=34)
    assert np.array_equal(out_c, out_p) and np.array_equal(lse_c, lse_p)
    assert_parity(out_p, lse_p, ro, rl, what="mla fp8 paged bitwise case")


def test_paged_config3_full_size_all_rows():
    announce("mla fp8 paged config3 full B64 H128 L4096, 16-row pages, every row")
    inp = W.make_mla_fp8_config(3)
    out, lse, ro, rl = run_paged(inp, 16, seed=35)
    err = assert_parity(out, lse, ro, rl, what="mla fp8 paged config3")
    print("paged config3 errors:", err)
