"""The MLA decode entry point that allocates nothing
(da_mla_decode_absorbed_noalloc, through the C ABI via the binding) against
the workspace entry point on the same inputs: two calls in a row, the second
with a smaller input, each bit-identical to da_mla_decode_absorbed (same
kernels, same plan) and within the bar of the fp64 oracle."""
import numpy as np
import pytest
import torch

import decode_attention_kv_bf16_amd as da
import workloads as W
from gpu_util import announce, assert_parity, mla_to_device
from oracle.attention import mla_absorbed_ref

pytestmark = pytest.mark.gpu


def f64(bits):
    return W.bf16_to_f32(bits).astype(np.float64)


def oracle(inp):
    outs, lses = [], []
    for b in range(len(inp.seq_lens)):
        L = int(inp.seq_lens[b])
        o, l = mla_absorbed_ref(f64(inp.q_nope[b:b + 1]), f64(inp.q_rope[b:b + 1]),
                                f64(inp.cache[b:b + 1, :max(L, 1)]), inp.seq_lens[b:b + 1],
                                f64(inp.w_uk), f64(inp.w_uv), inp.scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


CASES = [
    # the larger call first, then a smaller one over the same scratch
    (16, 128, [4096, 1, 0, 2000, 129, 4095, 77, 3000, 1024, 33, 2500, 4096, 0, 640, 1500, 2], 101),
    (3, 64, [700, 33, 5], 102),
]


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    assert da.lib().da_noalloc_scratch_bytes() == 64 << 20
    for B, H, lens, seed in CASES:
        announce(f"mla noalloc B{B} H{H} lens{lens}")
        inp = W.make_mla(B, H, lens, seed=seed, max_seq_len=max(lens) + 3, pad_value=float("nan"))
        qn, qr, cache, wuk, wuv, sl = mla_to_device(inp)
        out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        da.mla_decode_absorbed_noalloc(qn, qr, cache, wuk, wuv, sl, inp.scale, out=out, lse=lse)
        ref_out, ref_lse = da.mla_decode_absorbed(qn, qr, cache, wuk, wuv, sl, inp.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        ro, rl = oracle(inp)
        print("errors:", assert_parity(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, what=f"noalloc B{B}"))


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    announce("mla noalloc too large")
    # B = 512, L = 32768: the absorbed queries alone need 136 MiB
    qn = torch.zeros((512, 128, 128), dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros((512, 128, 64), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((1, 32768, 576), dtype=torch.bfloat16, device="cuda").expand(512, 32768, 576)
    w = torch.zeros((128, 512, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(da.DecodeAttnError) as e:
        da.mla_decode_absorbed_noalloc(qn, qr, cache, w, w)
    assert e.value.status == 3
