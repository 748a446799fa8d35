"""GPU parity of the GQA/MQA/MHA decode path (and the split-KV merge) against
the fp64 oracle, called through the C ABI via the Python binding.

Inputs come from workloads.py; rows past each sequence's length are filled
with NaN so that any out-of-range read poisons the result.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_bf16_amd as da
import workloads as W
from gpu_util import (announce, assert_parity, bf16_tensor, bf16_weight_bound, f32_tensor,
                      gqa_to_device)
from oracle.attention import combine_ref, gqa_decode_ref

pytestmark = pytest.mark.gpu

NAN = float("nan")


def oracle_rows(inp, seqs):
    """Oracle on a subset of sequences, one sequence per call (bounded memory
    at full size): returns (out, lse) for those rows only."""
    conv = (lambda a: W.bf16_to_f32(a).astype(np.float64)) if inp.dtype == "bf16" else \
        (lambda a: a.astype(np.float64))
    outs, lses = [], []
    for b in seqs:
        L = int(max(1, inp.seq_lens[b]))
        o, l = gqa_decode_ref(conv(inp.q[b:b + 1]), conv(inp.k[b:b + 1, :L]), conv(inp.v[b:b + 1, :L]),
                              inp.seq_lens[b:b + 1], inp.scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


def weight_bound(inp, seqs, ro, rl):
    """Per-row bound for kernels that round the softmax weights to bf16 for
    the value product on the matrix cores (bf16 caches)."""
    conv = (lambda a: W.bf16_to_f32(a).astype(np.float64)) if inp.dtype == "bf16" else \
        (lambda a: a.astype(np.float64))
    seqs = list(seqs)
    Lm = int(max(1, inp.seq_lens[seqs].max()))
    return bf16_weight_bound(conv(inp.q[seqs]), conv(inp.k[seqs, :Lm]), conv(inp.v[seqs, :Lm]),
                             inp.seq_lens[seqs], inp.scale, ro, rl)


def run(inp, num_splits=0, seq_lens=True):
    q, k, v, sl = gqa_to_device(inp)
    out, lse = da.gqa_decode(q, k, v, sl if seq_lens else None, inp.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def test_config1_tiny_fp32():
    announce("gqa config1 fp32 B1 Hq4 Hkv2 D64 L128")
    inp = W.make_gqa_config(1, pad_value=NAN)
    out, lse = run(inp)
    ro, rl = oracle_rows(inp, range(1))
    assert_parity(out, lse, ro, rl, what="config1")
    # fp32 inputs and fp32 accumulation: far inside the bar
    assert_parity(out, lse, ro, rl, out_rtol=1e-5, lse_atol=1e-5, what="config1 tight")


def test_config2_reduced_batch_all_rows():
    announce("gqa config2 shapes B4 Hq32 Hkv8 D128 L4096")
    inp = W.make_gqa_config(2, batch=4, pad_value=NAN)
    out, lse = run(inp)
    ro, rl = oracle_rows(inp, range(4))
    assert_parity(out, lse, ro, rl, what="config2 B4")
    assert_parity(out, lse, ro, rl, out_rtol=weight_bound(inp, range(4), ro, rl), lse_atol=1e-4,
                  what="config2 B4 tight")


def test_config2_full_size_all_rows():
    announce("gqa config2 full B32 L4096, every row")
    inp = W.make_gqa_config(2)
    out, lse = run(inp)
    ro, rl = oracle_rows(inp, range(32))
    assert_parity(out, lse, ro, rl, what="config2 full")


def test_config5_full_size_ragged_all_rows():
    announce("gqa config5 full ragged MHA B64 H32 D128 L<=8192 NaN-padded, every row")
    inp = W.make_gqa_config(5, pad_value=NAN)
    out, lse = run(inp)
    ro, rl = oracle_rows(inp, range(64))
    assert_parity(out, lse, ro, rl, what="config5 full")


EDGE = [
    # B, Hq, Hkv, D, lens, dtype
    (3, 8, 8, 128, [1, 1, 1], "bf16"),                 # L = 1
    (4, 8, 2, 128, [0, 5, 0, 17], "bf16"),             # empty sequences
    (8, 4, 1, 128, [1, 15, 16, 17, 255, 1023, 1025, 3000], "bf16"),   # ragged tails, MQA g=4
    (2, 32, 1, 128, [700, 2049], "bf16"),              # MQA g=32 (two head sub-groups)
    (2, 64, 4, 128, [333, 1], "bf16"),                 # g=16
    (2, 12, 4, 128, [100, 64], "bf16"),                # g=3
    (2, 16, 2, 64, [129, 4000], "bf16"),               # D=64, g=8
    (2, 6, 6, 64, [31, 2], "f32"),                     # fp32, D=64
    (2, 8, 4, 128, [513, 77], "f32"),                  # fp32, D=128
    (1, 14, 2, 128, [5000], "bf16"),                   # g=7
    (2, 8, 8, 128, [3000, 5000], "bf16"),              # 16 units: 16-wave workgroups, 16 splits
    (1, 32, 4, 128, [6000], "bf16"),                   # 8 heads per workgroup: 4-wave, 47 splits
    # units dividing the 256 CUs: 8-wave workgroups
    (16, 32, 8, 128, [4096, 1, 0, 2000, 129, 4095, 77, 3000,
                      1024, 33, 2500, 4096, 0, 640, 1500, 2], "bf16"),   # 128 units: 2 splits
    (256, 8, 1, 128, [(37 * i) % 301 for i in range(256)], "bf16"),     # 8 heads per workgroup, 1 split
    (32, 32, 8, 64, [(97 * i) % 700 + 1 for i in range(32)], "f32"),    # fp32, 1 split
    # 2048 workgroups, more than stay resident: sequences taken longest first,
    # with equal lengths (ties by index) and empty sequences
    (64, 32, 32, 128, [(i % 5) * 97 + (i % 3) for i in range(64)], "bf16"),
    # one long sequence: 128K rows over many splits and a ragged last step
    (1, 32, 8, 128, [131069], "bf16"),
]


@pytest.mark.parametrize("B,Hq,Hkv,D,lens,dtype", EDGE)
def test_edge_cases(B, Hq, Hkv, D, lens, dtype):
    announce(f"gqa edge B{B} Hq{Hq} Hkv{Hkv} D{D} lens{lens} {dtype}")
    inp = W.make_gqa(B, Hq, Hkv, D, lens, dtype, seed=11, max_seq_len=max(lens) + 7,
                     pad_value=NAN)
    out, lse = run(inp)
    ro, rl = oracle_rows(inp, range(B))
    assert_parity(out, lse, ro, rl, what="edge")


@pytest.mark.parametrize("splits", [1, 2, 7, 0, 64])
def test_split_count_invariance(splits):
    announce(f"gqa split invariance S={splits}")
    inp = W.make_gqa(3, 16, 4, 128, [2500, 1, 777], "bf16", seed=3, max_seq_len=2600,
                     pad_value=NAN)
    out, lse = run(inp, num_splits=splits)
    ro, rl = oracle_rows(inp, range(3))
    assert_parity(out, lse, ro, rl, what=f"S={splits}")
    assert_parity(out, lse, ro, rl, out_rtol=weight_bound(inp, range(3), ro, rl), lse_atol=1e-4,
                  what=f"S={splits} tight")
    # same split count: bitwise reproducible (no float atomics)
    out2, lse2 = run(inp, num_splits=splits)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (32, 8), (32, 32), (32, 1)])
def test_head_mapping_one_hot(Hq, Hkv):
    # V row one-hot on the KV head index: head h must return e_{h // g}
    announce(f"gqa head mapping Hq{Hq} Hkv{Hkv}")
    B, D, L = 2, 128, 300
    g = Hq // Hkv
    rng = np.random.default_rng(9)
    q = torch.from_numpy(rng.standard_normal((B, Hq, D)).astype(np.float32)).cuda().bfloat16()
    k = torch.from_numpy(rng.standard_normal((B, L, Hkv, D)).astype(np.float32)).cuda().bfloat16()
    v = torch.zeros((B, L, Hkv, D), dtype=torch.bfloat16, device="cuda")
    for kv in range(Hkv):
        v[:, :, kv, kv] = 1.0
    out, _ = da.gqa_decode(q, k, v)
    exp = np.zeros((Hq, D))
    for h in range(Hq):
        exp[h, h // g] = 1.0
    # the weights enter the value product in bf16 (relative error <= 2^-8
    # each): the weights of a one-hot column sum to 1 within 2^-8
    np.testing.assert_allclose(out.cpu().numpy(), np.broadcast_to(exp, (B, Hq, D)), atol=2.0 ** -8 + 1e-5)


def test_strided_query_and_no_seq_lens():
    announce("gqa strided q, seq_lens=None")
    inp = W.make_gqa(2, 8, 2, 128, [900, 900], "bf16", seed=4, max_seq_len=900)
    q, k, v, _ = gqa_to_device(inp)
    big = torch.zeros((2, 8, 3 * 128), dtype=torch.bfloat16, device="cuda")
    big[:, :, 128:256] = q
    qs = big[:, :, 128:256]
    assert not qs.is_contiguous()
    out, lse = da.gqa_decode(qs, k, v, None, inp.scale)
    ro, rl = oracle_rows(inp, range(2))
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, what="strided")


def test_error_codes_with_real_buffers():
    announce("gqa error codes")
    q = torch.zeros((2, 6, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 16, 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(da.DecodeAttnError) as e:
        da.gqa_decode(q, k, k)                  # 6 % 4 != 0
    assert e.value.status == 1
    q96 = torch.zeros((2, 4, 96), dtype=torch.bfloat16, device="cuda")
    k96 = torch.zeros((2, 16, 4, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(da.DecodeAttnError) as e:
        da.gqa_decode(q96, k96, k96)
    assert e.value.status == 2
    flat = torch.zeros(2 * 16 * 4 * 128 + 8, dtype=torch.bfloat16, device="cuda")
    kmis = flat[1:1 + 2 * 16 * 4 * 128].view(2, 16, 4, 128)   # 2-byte misaligned
    q4 = torch.zeros((2, 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(da.DecodeAttnError) as e:
        da.gqa_decode(q4, kmis, kmis)
    assert e.value.status == 1


@pytest.mark.parametrize("S,B,H,D", [(1, 2, 3, 128), (5, 4, 8, 128), (16, 3, 2, 64), (3, 2, 2, 512)])
def test_splitkv_combine_api(S, B, H, D):
    announce(f"combine S{S} B{B} H{H} D{D}")
    rng = np.random.default_rng(S * 100 + D)
    po = rng.standard_normal((S, B, H, D)).astype(np.float32)
    pl = (rng.standard_normal((S, B, H)) * 3).astype(np.float32)
    pl[rng.random((S, B, H)) < 0.3] = -np.inf      # empty splits
    pl[:, 0, 0] = -np.inf                           # a row with every split empty
    po[np.isneginf(pl)] = np.nan                     # never read
    out, lse = da.splitkv_combine(f32_tensor(po), f32_tensor(pl))
    ro, rl = combine_ref(po.astype(np.float64), pl.astype(np.float64))
    assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, out_rtol=1e-5, lse_atol=1e-5,
                  what="combine")


def test_split_pass_then_combine_equals_decode():
    announce("gqa split pass + combine == decode")
    inp = W.make_gqa(4, 32, 8, 128, [4096, 100, 2000, 3], "bf16", seed=8, max_seq_len=4096,
                     pad_value=NAN)
    q, k, v, sl = gqa_to_device(inp)
    po, pl = da.gqa_decode_split_pass(q, k, v, sl, inp.scale)
    assert po.shape[0] == da.gqa_num_splits(q, k) > 1
    out_c, lse_c = da.splitkv_combine(po, pl)
    out, lse = da.gqa_decode(q, k, v, sl, inp.scale)
    assert torch.equal(out, out_c) and torch.equal(lse, lse_c)
