"""GPU parity of the absorbed-MLA decode path against the fp64 oracle,
called through the C ABI via the Python binding.

Every check holds the bar: row-relative output error <= 1e-2 and
|lse error| <= 1e-3, for every sequence length from 1 row up. The kernel's
scores use the absorbed query rounded to bf16; the library corrects each lse
by the first-order effect of that rounding, so short sequences (where the
score shifts of a few rows do not average out) meet the same bar as long ones.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_bf16_amd as da
import workloads as W
from gpu_util import announce, assert_parity, mla_to_device, row_rel_err
from oracle.attention import mla_absorbed_ref

pytestmark = pytest.mark.gpu

NAN = float("nan")


def f64(bits):
    return W.bf16_to_f32(bits).astype(np.float64)


def oracle_rows(inp, seqs):
    """The oracle one sequence at a time (bounded memory), stacked."""
    wuk, wuv = f64(inp.w_uk), f64(inp.w_uv)
    outs, lses = [], []
    for b in seqs:
        L = int(inp.seq_lens[b])
        o, l = mla_absorbed_ref(f64(inp.q_nope[b:b + 1]), f64(inp.q_rope[b:b + 1]),
                                f64(inp.cache[b:b + 1, :max(L, 1)]), inp.seq_lens[b:b + 1], wuk, wuv,
                                inp.scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


def run(inp, num_splits=0):
    qn, qr, cache, wuk, wuv, sl = mla_to_device(inp)
    out, lse = da.mla_decode_absorbed(qn, qr, cache, wuk, wuv, sl, inp.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def test_config3_reduced_batch_all_rows():
    announce("mla config3 shapes B4 H128 L4096")
    inp = W.make_mla_config(3, batch=4, pad_value=NAN)
    out, lse = run(inp)
    ro, rl = oracle_rows(inp, range(4))
    err = assert_parity(out, lse, ro, rl, what="config3 B4")
    print("config3 B4 max row rel err, max lse err:", err)


def test_config3_full_size_all_rows():
    announce("mla config3 full B64 H128 L4096, every row")
    inp = W.make_mla_config(3)
    out, lse = run(inp)
    ro, rl = oracle_rows(inp, range(64))
    err = assert_parity(out, lse, ro, rl, what="config3 full")
    print("config3 full max row rel err, max lse err:", err)


def test_config4_long_context_all_rows():
    announce("mla config4 full B4 H128 L~U[16384,32768] NaN-padded")
    inp = W.make_mla_config(4, pad_value=NAN)
    out, lse = run(inp)
    ro, rl = oracle_rows(inp, range(4))
    err = assert_parity(out, lse, ro, rl, what="config4")
    print("config4 max row rel err, max lse err:", err, "lens", inp.seq_lens)


def assert_all(inp, out, lse, what, seqs=None):
    seqs = list(range(len(inp.seq_lens)) if seqs is None else seqs)
    ro, rl = oracle_rows(inp, seqs)
    return assert_parity(out[seqs], lse[seqs], ro, rl, what=what)


EDGE = [
    # B, H, lens
    (4, 128, [1, 2, 31, 33]),
    (3, 128, [0, 32, 0]),            # empty sequences
    (2, 64, [100, 1000]),
    (2, 32, [65, 7]),
    (3, 16, [300, 1, 4097]),
    (5, 128, [2048, 17, 4000, 129, 64]),
    (2, 48, [700, 33]),              # three-wave shapes
    (3, 96, [1500, 2, 260]),
    (2, 128, [0, 0]),                # nothing to attend to at all
    (7, 128, [1, 5000, 0, 33, 12000, 64, 2]),   # lengths spread over 4 orders
    (1, 128, [65533]),               # one long sequence over every workgroup
]


@pytest.mark.parametrize("B,H,lens", EDGE)
def test_edge_cases(B, H, lens):
    announce(f"mla edge B{B} H{H} lens{lens}")
    inp = W.make_mla(B, H, lens, seed=21, max_seq_len=max(lens) + 5, pad_value=NAN)
    out, lse = run(inp)
    print("errors:", assert_all(inp, out, lse, what=f"edge {lens}"))


@pytest.mark.parametrize("splits", [1, 2, 5, 0, 40])
def test_split_count_invariance(splits):
    announce(f"mla split invariance S={splits}")
    inp = W.make_mla(2, 128, [3000, 1200], seed=5, max_seq_len=3001, pad_value=NAN)
    out, lse = run(inp, num_splits=splits)
    ro, rl = oracle_rows(inp, range(2))
    err = assert_parity(out, lse, ro, rl, what=f"S={splits}")
    print(f"S={splits} errors:", err)
    out2, lse2 = run(inp, num_splits=splits)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_balanced_splits_over_many_sequences():
    # 300 ragged sequences of 16 heads: the device-side split planner scans
    # the lengths 64 at a time, so this covers several of its chunks, empty
    # sequences in between and one sequence far longer than the rest
    announce("mla balanced splits B300 H16 ragged")
    rng = np.random.default_rng(8)
    lens = rng.integers(0, 900, 300)
    lens[::37] = 0
    lens[5] = 1200
    inp = W.make_mla(300, 16, lens, seed=9, max_seq_len=1201, pad_value=NAN)
    qn, qr, cache, _, wuv, _ = mla_to_device(inp)
    assert da.mla_num_splits(qn, qr, cache, wuv) == 0      # balanced on the device
    del qn, qr, cache, wuv
    p_out, p_lse = run(inp)
    print(assert_all(inp, p_out, p_lse, what="B300"))


def test_stages_compose_to_the_full_call():
    announce("mla stages compose")
    inp = W.make_mla(3, 128, [1500, 40, 3000], seed=6, max_seq_len=3000, pad_value=NAN)
    qn, qr, cache, wuk, wuv, sl = mla_to_device(inp)
    absorb, attend, merge, out_s, lse_s, _ = da.mla_stages(qn, qr, cache, wuk, wuv, sl, inp.scale)
    absorb()
    attend()
    merge()
    out, lse = da.mla_decode_absorbed(qn, qr, cache, wuk, wuv, sl, inp.scale)
    assert torch.equal(out, out_s) and torch.equal(lse, lse_s)


@pytest.mark.parametrize("H", [32, 64, 96, 128])   # 1 to 4 waves of 32 heads
def test_balanced_splits_with_poisoned_partials(H):
    """Balanced splits over the 32-head-block kernel, with sequences of 2,
    32, 1, 75, 14 and 125 splits of 5 tiles on 256 workgroups. The partial
    buffers (and the split table after the lse slots) start as NaN, the
    attention stage runs twice, and the stages must still equal the one-call
    path bit for bit and the oracle to the bar: the merge reads only what the
    latest attention stage wrote."""
    announce(f"mla balanced splits, poisoned partials H{H}")
    lens = [300, 5000, 17, 12000, 2100, 20000]
    inp = W.make_mla(len(lens), H, lens, seed=21, max_seq_len=20000, pad_value=NAN)
    qn, qr, cache, wuk, wuv, sl = mla_to_device(inp)
    assert da.mla_num_splits(qn, qr, cache, wuv) == 0
    absorb, attend, merge, out_s, lse_s, bufs = da.mla_stages(qn, qr, cache, wuk, wuv, sl, inp.scale)
    bufs["part_out"].fill_(0xFF)                 # bf16 0xFFFF: NaN
    bufs["part_lse"].fill_(NAN)
    absorb()
    attend()
    attend()
    merge()
    out, lse = da.mla_decode_absorbed(qn, qr, cache, wuk, wuv, sl, inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out_s) and torch.equal(lse, lse_s)
    print(assert_all(inp, out.cpu().numpy(), lse.cpu().numpy(), what=f"mla balanced poisoned H{H}"))


@pytest.mark.parametrize("B", [5, 20])   # one 16-row merge block (two thread groups per row), two blocks
def test_empty_fixed_splits_are_never_read(B):
    """Fixed splits past a sequence's end write lse -inf and no pieces; the
    merge must not read their slots. The partial buffers are filled with NaN
    before the attention stage, so any read of an empty slot shows."""
    announce(f"mla empty fixed splits B{B}")
    lens = [2048, 17, 4000, 129, 64] * (B // 5)
    inp = W.make_mla(B, 128, lens, seed=8, max_seq_len=4000, pad_value=NAN)
    qn, qr, cache, wuk, wuv, sl = mla_to_device(inp)
    absorb, attend, merge, out, lse, bufs = da.mla_stages(qn, qr, cache, wuk, wuv, sl, inp.scale,
                                                          num_splits=3)
    bufs["part_out"].fill_(0xFF)                 # bf16 0xFFFF: NaN
    bufs["part_lse"].fill_(float("nan"))
    absorb()
    attend()
    merge()
    torch.cuda.synchronize()
    ro, rl = oracle_rows(inp, range(B))
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, what="mla empty fixed splits")


def test_identity_projection_reduces_to_mqa():
    # W_UK, W_UV = selection of the first 128 latent columns, q_rope = 0:
    # absorbed MLA becomes MQA over K = V = c_kv[:, :128] with 128 heads sharing it
    announce("mla with selection matrices vs gqa kernel (MQA)")
    B, H, L = 2, 128, 700
    inp = W.make_mla(B, H, [L, 300], seed=7, max_seq_len=L)
    sel = np.zeros((H, 512, 128), np.float32)
    sel[:, np.arange(128), np.arange(128)] = 1.0
    inp.w_uk = W.bf16_round(sel)
    inp.w_uv = W.bf16_round(sel)
    inp.q_rope = np.zeros_like(inp.q_rope)
    out, lse = run(inp)
    # the same problem through the GQA kernel: Hq = 128 heads on one KV head
    c = torch.from_numpy(inp.cache[:, :, :128].copy().view(np.int16)).cuda().view(torch.bfloat16)
    kv = c[:, :, None, :].contiguous()
    q = torch.from_numpy(inp.q_nope.view(np.int16)).cuda().view(torch.bfloat16)
    sl = torch.from_numpy(inp.seq_lens).cuda()
    o2, l2 = da.gqa_decode(q, kv, kv, sl, inp.scale)
    # the GQA kernel keeps q exact; MLA rounds P and o~ to bf16
    err = row_rel_err(out, o2.cpu().numpy().astype(np.float64))
    assert err.max() < 1e-2
    assert np.abs(lse - l2.cpu().numpy()).max() < 1e-3


def test_error_codes_with_real_buffers():
    announce("mla error codes")
    qn = torch.zeros((2, 24, 128), dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros((2, 24, 64), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((2, 16, 576), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((24, 512, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(da.DecodeAttnError) as e:
        da.mla_decode_absorbed(qn, qr, cache, w, w)     # 24 heads: not a multiple of 16
    assert e.value.status == 2


def test_late_dominant_row_forces_reference_restart():
    # A row near the end of a split whose score for one head exceeds the first
    # tile's maximum by far more than 2^64: the kernel must restart that split
    # with a raised reference and still match the oracle.
    announce("mla late dominant row (reference restart)")
    B, H, L = 2, 128, 1500
    inp = W.make_mla(B, H, [L, 900], seed=12, max_seq_len=L, pad_value=NAN)
    qr = W.bf16_to_f32(inp.q_rope[0, 5])
    row = W.bf16_to_f32(inp.cache[0, L - 3]).copy()
    row[512:] = 40.0 * qr                      # score ~ 40 |q_rope|^2 / sqrt(192) ~ 180 nats
    inp.cache[0, L - 3] = W.bf16_round(row)
    out, lse = run(inp, num_splits=1)
    ro, rl = oracle_rows(inp, range(B))
    assert rl[0, 5] > 100                      # the planted row dominates head 5
    # one row carries almost all the weight (no averaging of score errors)
    print("errors:", assert_parity(out, lse, ro, rl, what="late dominant row"))
