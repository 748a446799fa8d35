"""The C ABI on the host: the library loads, exports every declared symbol,
its structs match the binding, planning answers, and bad arguments are
rejected on the host before anything is launched.

Argument-rejection cases pass fake (never dereferenced) pointers, so they are
skipped on a machine with a GPU, where the GPU tests cover the same errors
with real buffers.
"""
import ctypes
import os
import re

import pytest
import torch

import decode_attention_kv_bf16_amd as da

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_attn.h")

needs_lib = pytest.mark.skipif(not os.path.exists(da.LIB_PATH), reason="library not built")
cpu_only = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer checks run on CPU only")


def declared_symbols():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"DA_EXPORT\s+[\w\s\*]+?\b(da_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ("da_gqa_decode", "da_mla_decode_absorbed", "da_splitkv_combine",
                 "da_gqa_decode_workspace_size", "da_mla_decode_workspace_size",
                 "da_status_string"):
        assert name in syms


@needs_lib
def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(da.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(L, name), name
    # and the binding knows all of them
    assert set(declared_symbols()) == set(da._SIGNATURES)


@needs_lib
def test_struct_mirrors_and_version():
    L = da.lib()
    assert L.da_gqa_params_size() == ctypes.sizeof(da.GqaParams) == 80
    assert L.da_mla_params_size() == ctypes.sizeof(da.MlaParams)
    assert L.da_paged_kv_size() == ctypes.sizeof(da.PagedKv) == 24
    assert L.da_kv_scales_size() == ctypes.sizeof(da.KvScales) == 40
    assert L.da_append_size() == ctypes.sizeof(da.Append) == 40
    assert L.da_version() >= 100
    for s, txt in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported configuration"),
                   (3, b"workspace too small"), (4, b"HIP runtime error"), (99, b"unknown status")]:
        assert L.da_status_string(s) == txt


def gqa(B=32, Hq=32, Hkv=8, D=128, L=4096, dtype=da.DA_DTYPE_BF16, splits=0):
    p = da.GqaParams()
    p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.max_seq_len = B, Hq, Hkv, D, L
    p.dtype = dtype
    p.softmax_scale = D ** -0.5
    p.q_stride_b, p.q_stride_h = Hq * D, D
    p.kv_stride_b, p.kv_stride_t, p.kv_stride_h = L * Hkv * D, Hkv * D, D
    p.num_splits = splits
    return p


def mla(B=64, H=128, L=4096, splits=0):
    p = da.MlaParams()
    p.batch, p.num_heads, p.kv_lora_rank, p.qk_rope_dim = B, H, 512, 64
    p.qk_nope_dim, p.v_head_dim, p.max_seq_len = 128, 128, L
    p.softmax_scale = 192 ** -0.5
    p.cache_stride_b, p.cache_stride_t = L * 576, 576
    p.num_splits = splits
    return p


@needs_lib
@cpu_only
def split_cost_model(units, length, slots, min_rows, overhead):
    # the planner's rule, written out: fewest rounds x (chunk + fixed cost)
    best = None
    for s in range(1, min(-(-length // min_rows), 1024) + 1):
        cost = -(-units * s // slots) * (-(-length // s) + overhead)
        if best is None or cost < best[1]:
            best = (s, cost)
    return best[0]


def test_split_planning_without_a_device():
    # with no device the planner assumes a full MI355X (256 CUs) and, for
    # MLA, an occupancy of 1 workgroup per CU
    L = da.lib()
    n = lambda p: L.da_gqa_decode_num_splits(ctypes.byref(p))
    ws = lambda p: L.da_gqa_decode_workspace_size(ctypes.byref(p))
    # GQA, with units = (b, kv head, head group): >= 2 per CU -> one split;
    # units dividing the CUs (CUs / units = 1 or 2) -> 8-wave workgroups that
    # fill the CUs once; otherwise >= half a CU's worth -> 4-wave workgroups,
    # 2 per CU; fewer -> 16-wave workgroups, one per CU; chunks no shorter
    # than 128 rows
    assert n(gqa()) == 1                                   # Llama-3-8B: 256 units -> 256 8-wave workgroups
    assert ws(gqa()) == 0                                  # one split: no partials
    assert n(gqa(64, 32, 32, 128, 8192)) == 1              # ragged MHA: 2048 units
    assert n(gqa(16, 32, 8, 128, 4096)) == 2               # 128 units -> 8-wave, 2 splits
    assert ws(gqa(16, 32, 8, 128, 4096)) == 2 * 16 * 32 * 128 * 4 + 2 * 16 * 32 * 4
    assert n(gqa(24, 32, 8, 128, 4096)) == 3               # 192 units -> 4-wave, 2 per CU
    assert n(gqa(48, 32, 8, 128, 4096)) == 2               # 384 units -> 4-wave, 2 per CU
    assert n(gqa(4, 32, 8, 128, 4096)) == 8                # 32 units -> 16-wave, 8 splits
    assert n(gqa(8, 8, 1, 128, 4096)) == 32                # MQA B=8: 8 units (8 heads: 4-wave), 128-row floor
    assert n(gqa(1, 4, 2, 64, 128, da.DA_DTYPE_F32)) == 1  # tiny: one split, no workspace
    assert ws(gqa(1, 4, 2, 64, 128, da.DA_DTYPE_F32)) == 0
    assert n(gqa(splits=7)) == 7
    assert n(gqa(L=5, splits=9)) == 5                      # never more splits than rows
    m = lambda p: L.da_mla_decode_num_splits(ctypes.byref(p))
    # MLA: a batch below the resident workgroups (256) is split on the device
    # by the actual lengths (0 = balanced); from 256 sequences on, fixed splits
    assert m(mla()) == 0                                   # DeepSeek-V3 B=64
    assert m(mla(4, 128, 32768)) == 0
    assert m(mla(512, 128, 4096)) == split_cost_model(512, 4096, 256, 128, 128) == 1
    assert m(mla(256, 128, 32768)) == split_cost_model(256, 32768, 256, 128, 128)
    assert m(mla(splits=3)) == 3                           # forced: fixed splits
    assert m(mla(H=80)) == -1                              # invalid
    assert L.da_mla_decode_workspace_size(ctypes.byref(mla())) >= 64 * 128 * 576 * 2


def mla_partials(p):
    po, pl = ctypes.c_size_t(), ctypes.c_size_t()
    st = da.lib().da_mla_partials_size(ctypes.byref(p), ctypes.byref(po), ctypes.byref(pl))
    return st, po.value, pl.value


@needs_lib
@cpu_only
def test_mla_partials_size_without_a_device():
    L = da.lib()
    up = lambda n: -(-n // 256) * 256
    # fixed splits: S * B slots of H rows (bf16 o~ of 512, float lse)
    st, po, pl = mla_partials(mla(64, 128, 4096, splits=3))
    assert st == 0 and po == up(3 * 64 * 128 * 512 * 2) and pl == up(3 * 64 * 128 * 4)
    # balanced: at most (resident workgroups + B) slots, then 2 int32 per
    # sequence for the table of each sequence's slots
    st, po, pl = mla_partials(mla(64, 128, 4096))
    assert st == 0 and po == up((256 + 64) * 128 * 512 * 2)
    assert pl == up((256 + 64) * 128 * 4) + up(64 * 2 * 4)
    # the workspace is the absorbed-query buffer (q^ of 576 and q~_lo of 512
    # bf16 per row) followed by the two partial buffers
    for p in (mla(), mla(splits=3), mla(4, 16, 100)):
        _, po, pl = mla_partials(p)
        assert L.da_mla_decode_workspace_size(ctypes.byref(p)) == up(p.batch * p.num_heads * 1088 * 2) + po + pl
    assert mla_partials(mla(H=80))[0] == 2
    assert L.da_mla_partials_size(ctypes.byref(mla()), None, None) == 1


FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
FAKE_MIS = ctypes.c_void_p(0x10002)   # misaligned


def call_gqa(p, q=FAKE, k=FAKE, v=FAKE, sl=None, out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 40):
    return da.lib().da_gqa_decode(ctypes.byref(p) if p is not None else None, q, k, v, sl, out,
                                  lse, ws, ws_bytes, None)


@needs_lib
@cpu_only
@pytest.mark.parametrize("mutate,code", [
    (lambda p: setattr(p, "num_kv_heads", 3), 1),       # 32 % 3 != 0: the pages' assert
    (lambda p: setattr(p, "head_dim", 96), 2),
    (lambda p: setattr(p, "head_dim", 0), 1),
    (lambda p: setattr(p, "batch", 0), 1),
    (lambda p: setattr(p, "max_seq_len", 0), 1),
    (lambda p: setattr(p, "num_splits", -1), 1),
    (lambda p: setattr(p, "dtype", 7), 1),
    (lambda p: setattr(p, "kv_stride_t", 1028), 1),      # not a multiple of 16 bytes
    (lambda p: setattr(p, "q_stride_h", -128), 1),
    (lambda p: setattr(p, "softmax_scale", float("nan")), 1),
])
def test_gqa_rejects_bad_parameters(mutate, code):
    p = gqa()
    mutate(p)
    assert call_gqa(p) == code
    assert da.lib().da_gqa_decode_workspace_size(ctypes.byref(p)) == 0


@needs_lib
@cpu_only
def test_gqa_rejects_bad_pointers_and_workspace():
    p = gqa(16, 32, 8, 128, 4096)        # planned with 2 splits: needs a workspace
    assert da.lib().da_gqa_decode_workspace_size(ctypes.byref(p)) > 0
    assert call_gqa(None) == 1
    assert call_gqa(p, q=None) == 1
    assert call_gqa(p, out=None) == 1
    assert call_gqa(p, k=FAKE_MIS) == 1
    assert call_gqa(p, sl=ctypes.c_void_p(0x10001)) == 1
    assert call_gqa(p, ws=None) == 3
    assert call_gqa(p, ws_bytes=100) == 3
    assert call_gqa(p, ws=FAKE_MIS) == 1


@needs_lib
@cpu_only
def test_mla_and_combine_reject_bad_parameters():
    L = da.lib()

    def call_mla(p, ws_bytes=1 << 40, ptr=FAKE):
        return L.da_mla_decode_absorbed(ctypes.byref(p), ptr, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                        None, FAKE, ws_bytes, None)
    for field, val, code in [("kv_lora_rank", 256, 2), ("qk_rope_dim", 32, 2), ("num_heads", 24, 2),
                             ("num_heads", 256, 2), ("num_heads", 80, 2), ("num_heads", 112, 2), ("batch", 0, 1), ("cache_stride_t", 512, 1),
                             ("max_seq_len", -1, 1), ("softmax_scale", 0.0, 2), ("softmax_scale", -0.1, 2),
                             ("softmax_scale", float("nan"), 1)]:
        p = mla()
        setattr(p, field, val)
        assert call_mla(p) == code, field
    assert call_mla(mla(), ws_bytes=10) == 3
    assert call_mla(mla(), ptr=FAKE_MIS) == 1
    assert call_mla(mla(), ptr=None) == 1
    comb = L.da_splitkv_combine
    assert comb(0, 1, 1, 128, FAKE, FAKE, FAKE, None, None) == 1
    assert comb(2, 1, 1, 126, FAKE, FAKE, FAKE, None, None) == 1
    assert comb(2, 1, 1, 2048, FAKE, FAKE, FAKE, None, None) == 1
    assert comb(2, 1, 1, 128, None, FAKE, FAKE, None, None) == 1
    assert comb(2, 1, 1, 128, FAKE_MIS, FAKE, FAKE, None, None) == 1


def paging(table=FAKE, page_size=16, max_blocks=256, page_stride=16 * 8 * 128):
    pg = da.PagedKv()
    pg.block_table = table.value if table is not None else None
    pg.page_size, pg.max_blocks_per_seq, pg.page_stride = page_size, max_blocks, page_stride
    return pg


@needs_lib
@cpu_only
@pytest.mark.parametrize("kw", [
    dict(table=None),                          # no block table
    dict(table=ctypes.c_void_p(0x10002)),      # misaligned table
    dict(page_size=8),                         # below 16 rows
    dict(page_size=48),                        # not a power of two
    dict(page_size=1 << 21),                   # too large
    dict(max_blocks=255),                      # 255 * 16 < 4096 rows
    dict(page_stride=0),
    dict(page_stride=4),                       # 8 bytes: not a 16-byte multiple
])
def test_paged_entry_points_reject_bad_paging(kw):
    L = da.lib()
    p = gqa(32, 32, 8, 128, 4096)
    pg = paging(**kw)
    assert L.da_gqa_decode_paged(ctypes.byref(p), ctypes.byref(pg), FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, FAKE, 1 << 40, None) == 1
    m = mla(64, 128, 4096)
    pgm = paging(**{"page_stride": 16 * 576, **kw})
    assert L.da_mla_decode_absorbed_paged(ctypes.byref(m), ctypes.byref(pgm), FAKE, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 1
    assert L.da_mla_attend_split_pass_paged(ctypes.byref(m), ctypes.byref(pgm), FAKE, FAKE, FAKE,
                                            FAKE, FAKE, None) == 1


@needs_lib
@cpu_only
def test_paged_entry_points_reject_missing_descriptor_and_workspace():
    L = da.lib()
    p = gqa(16, 32, 8, 128, 4096)        # 2 splits: needs a workspace
    assert L.da_gqa_decode_paged(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 1 << 40, None) == 1
    pg = paging()
    assert L.da_gqa_decode_paged(ctypes.byref(p), ctypes.byref(pg), FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, None, 0, None) == 3
    m = mla(64, 128, 4096)
    pgm = paging(page_stride=16 * 576)
    assert L.da_mla_decode_absorbed_paged(ctypes.byref(m), None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 1
    assert L.da_mla_decode_absorbed_paged(ctypes.byref(m), ctypes.byref(pgm), FAKE, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, None) == 3


def fp8_params(B=32, Hq=32, Hkv=8, D=128, L=4096):
    p = gqa(B, Hq, Hkv, D, L)
    p.dtype = da.DA_DTYPE_FP8_E4M3
    p.kv_stride_b, p.kv_stride_t, p.kv_stride_h = L * Hkv * D, Hkv * D, D     # bytes
    return p


def scales(k=FAKE, v=FAKE, sb=4096 * 8, st=8, sh=1):
    s = da.KvScales()
    s.k_scale = k.value if k is not None else None
    s.v_scale = v.value if v is not None else None
    s.stride_b, s.stride_t, s.stride_h = sb, st, sh
    return s


@needs_lib
def test_fp8_params_plan_like_bf16():
    L = da.lib()
    p = fp8_params()
    assert L.da_gqa_decode_num_splits(ctypes.byref(p)) == L.da_gqa_decode_num_splits(ctypes.byref(gqa()))
    p.kv_stride_t = 8 * 128 + 8          # 1032 bytes: not a multiple of 16
    assert L.da_gqa_decode_num_splits(ctypes.byref(p)) == 0


@needs_lib
@cpu_only
def test_fp8_entry_point_rejects_bad_arguments():
    L = da.lib()

    def call(p, s, ws_bytes=1 << 40):
        return L.da_gqa_decode_fp8(ctypes.byref(p), ctypes.byref(s) if s is not None else None, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)
    assert call(fp8_params(), None) == 1                       # no scales
    assert call(fp8_params(), scales(k=None)) == 1
    assert call(fp8_params(), scales(v=ctypes.c_void_p(0x10002))) == 1   # misaligned
    assert call(fp8_params(), scales(st=-8)) == 1
    bf = gqa()
    assert call(bf, scales()) == 1                             # not the fp8 dtype
    p = fp8_params()
    p.q_stride_h = 132                                         # 264 bytes of bf16 q
    assert call(p, scales()) == 1
    p16 = fp8_params(16)                                       # two splits: needs a workspace
    assert call(p16, scales(), ws_bytes=0) == 3
    # the entry points without scales refuse the fp8 dtype
    assert L.da_gqa_decode(ctypes.byref(fp8_params()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           1 << 40, None) == 1
    assert L.da_gqa_decode_split_pass(ctypes.byref(fp8_params()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      None) == 1


def mla_scales(n=FAKE, r=FAKE, sb=4096, st=1):
    s = da.MlaScales()
    s.nope_scale, s.rope_scale, s.stride_b, s.stride_t = n, r, sb, st
    return s


@needs_lib
@cpu_only
def test_mla_fp8_entry_point_rejects_bad_arguments():
    L = da.lib()

    def call(p, s, ws_bytes=1 << 40, codes=FAKE):
        return L.da_mla_decode_absorbed_fp8(ctypes.byref(p), ctypes.byref(s) if s is not None else None,
                                            FAKE, FAKE, codes, None, FAKE, FAKE, FAKE, None, FAKE,
                                            ws_bytes, None)
    # the same workspace layout as the bf16 call for these shapes
    assert L.da_mla_decode_fp8_workspace_size(ctypes.byref(mla())) > 0
    assert call(mla(), None) == 1                              # no scales
    assert call(mla(), mla_scales(n=None)) == 1
    assert call(mla(), mla_scales(r=ctypes.c_void_p(0x10002))) == 1   # misaligned
    assert call(mla(), mla_scales(st=-1)) == 1
    assert call(mla(), mla_scales(sb=-1)) == 1
    assert call(mla(), mla_scales(st=(1 << 24) + 1)) == 1      # token stride beyond 2^24
    assert call(mla(), mla_scales(), codes=None) == 1
    assert call(mla(), mla_scales(), codes=FAKE_MIS) == 1
    assert call(mla(), mla_scales(), ws_bytes=10) == 3
    p = mla()
    p.cache_stride_t = 584                                     # bytes: not a multiple of 16
    assert call(p, mla_scales()) == 1
    assert L.da_mla_decode_fp8_workspace_size(ctypes.byref(p)) == 0
    p.cache_stride_t = 592                                     # 16-byte multiple: fine in bytes
    assert L.da_mla_decode_fp8_workspace_size(ctypes.byref(p)) > 0
    for field, val, code in [("kv_lora_rank", 256, 2), ("num_heads", 24, 2), ("batch", 0, 1),
                             ("softmax_scale", 0.0, 2)]:
        p = mla()
        setattr(p, field, val)
        assert call(p, mla_scales()) == code, field
    # paged pools: the descriptor is required and checked like the other paged calls
    def call_paged(p, pg, s=mla_scales()):
        return L.da_mla_decode_absorbed_fp8_paged(ctypes.byref(p), ctypes.byref(pg) if pg is not None else None,
                                                  ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                  None, FAKE, 1 << 40, None)
    mp = mla()
    mp.cache_stride_b = 0
    assert call_paged(mp, None) == 1
    assert call_paged(mp, paging(page_size=48, page_stride=16 * 576)) == 1        # not a power of two
    assert call_paged(mp, paging(max_blocks=255, page_stride=16 * 576)) == 1      # too few blocks
    assert call_paged(mp, paging(page_stride=16 * 576 + 8)) == 1                  # not a 16-byte multiple
    assert call_paged(mp, paging(page_stride=16 * 576), mla_scales(st=-1)) == 1
    # the GQA fp8 call bounds its token stride the same way
    assert L.da_gqa_decode_fp8(ctypes.byref(fp8_params()), ctypes.byref(scales(st=(1 << 24) + 8)), FAKE,
                               FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 1


@needs_lib
def test_sliding_window_planning_without_a_device():
    L = da.lib()
    full = gqa(B=2, Hq=8, Hkv=2)
    bad = gqa(B=2, Hq=8, Hkv=2)
    bad.sliding_window = -1
    assert L.da_gqa_decode_num_splits(ctypes.byref(bad)) == 0
    assert L.da_gqa_decode(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 1
    s_full = L.da_gqa_decode_num_splits(ctypes.byref(full))
    for w in (1, 16, 100, 1000, 4081, 4096, 1 << 20):
        p = gqa(B=2, Hq=8, Hkv=2)
        p.sliding_window = w
        s = L.da_gqa_decode_num_splits(ctypes.byref(p))
        assert 1 <= s <= s_full
        # planned on min(L_max, w + 15) rows: the splits cover them
        assert L.da_gqa_decode_workspace_size(ctypes.byref(p)) <= L.da_gqa_decode_workspace_size(ctypes.byref(full))


def append_desc(r=128, style=0, base=10000.0, inv=None, sb=48 * 128, sh=128):
    ap = da.Append()
    ap.rotary_dim, ap.rope_style, ap.rope_base, ap.inv_freq = r, style, base, inv
    ap.new_stride_b, ap.new_stride_h = sb, sh
    return ap


@needs_lib
@pytest.mark.parametrize("kw,code", [
    ({"r": 0}, 1), ({"r": 12}, 1), ({"r": 136}, 1), ({"style": 2}, 1), ({"base": 1.0}, 1),
    ({"base": float("nan")}, 1), ({"base": float("inf")}, 1), ({"inv": 0x10002}, 1),
    ({"sb": -128}, 1), ({"sh": 4}, 1),
])
def test_append_rejects_bad_descriptors(kw, code):
    L = da.lib()
    ap = append_desc(**kw)
    assert L.da_gqa_append_rope(ctypes.byref(gqa()), ctypes.byref(ap), None, FAKE, FAKE, FAKE, FAKE,
                                FAKE, FAKE, FAKE, None) == code
    mla_ap = append_desc(**{**{"r": 64, "sb": 576, "sh": 0}, **kw})
    assert L.da_mla_append_rope(ctypes.byref(mla()), ctypes.byref(mla_ap), None, FAKE, FAKE, FAKE,
                                FAKE, FAKE, None) == code


@needs_lib
def test_append_rejects_bad_buffers_and_dtypes():
    L = da.lib()
    ok = append_desc()

    def gcall(p=None, ap=ok, pages=None, ptrs=None):
        ptrs = ptrs or [FAKE] * 7
        return L.da_gqa_append_rope(ctypes.byref(p or gqa()), None if ap is None else ctypes.byref(ap),
                                    pages, *ptrs, None)
    assert gcall(ap=None) == 1
    assert gcall(p=gqa(dtype=da.DA_DTYPE_FP8_E4M3)) == 2            # no fp8 append
    assert gcall(ptrs=[FAKE, None] + [FAKE] * 5) == 1               # no q_out
    assert gcall(ptrs=[FAKE] * 4 + [ctypes.c_void_p(0x10002)] + [FAKE] * 2) == 1   # positions misaligned
    assert gcall(ptrs=[FAKE] * 5 + [ctypes.c_void_p(0x10008), FAKE]) == 1          # cache misaligned
    pg = da.PagedKv()
    pg.block_table, pg.page_size, pg.max_blocks_per_seq, pg.page_stride = FAKE.value, 24, 256, 16 * 8 * 128
    assert gcall(pages=ctypes.byref(pg)) == 1                       # page size not a power of two
    assert L.da_mla_append_rope(ctypes.byref(mla()), ctypes.byref(append_desc(r=128, sb=576, sh=0)),
                                None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1   # r > 64


@needs_lib
def test_fp8_append_rejects_bad_arguments():
    L = da.lib()

    def sc(st=8, sh=1, k=FAKE):
        s = da.KvScales()
        s.k_scale, s.v_scale = k.value if k is not None else None, FAKE.value
        s.stride_b, s.stride_t, s.stride_h = 4096 * 8, st, sh
        return s

    def call(p, scales, pages=None, ap=None):
        ap = ap or append_desc()
        return L.da_gqa_append_rope_fp8(ctypes.byref(p), ctypes.byref(ap), pages,
                                        None if scales is None else ctypes.byref(scales),
                                        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    f8 = gqa(dtype=da.DA_DTYPE_FP8_E4M3)
    f8.kv_stride_b, f8.kv_stride_t, f8.kv_stride_h = 4096 * 8 * 128, 8 * 128, 128
    assert call(gqa(), sc()) == 1                                  # not the fp8 dtype
    assert call(f8, None) == 1                                     # no scales
    assert call(f8, sc(k=None)) == 1
    assert call(f8, sc(st=8, sh=0)) == 2                           # dynamic per-token, shared by heads
    assert call(f8, sc(st=-8)) == 1
    pg = da.PagedKv()
    pg.block_table, pg.page_size, pg.max_blocks_per_seq, pg.page_stride = FAKE.value, 16, 256, 16 * 8 * 128
    assert call(f8, sc(), pages=ctypes.byref(pg)) == 2             # no paged E4M3 pools
    assert call(f8, sc(), ap=append_desc(r=12)) == 1


@needs_lib
def test_fp8_paged_rejects_small_pages_and_per_page_scales():
    L = da.lib()
    f8 = gqa(dtype=da.DA_DTYPE_FP8_E4M3)
    f8.kv_stride_b, f8.kv_stride_t, f8.kv_stride_h = 0, 8 * 128, 128

    def call(ps=32, sb=32 * 8, st=8, p=f8, pages=True, scales=True):
        pg = da.PagedKv()
        pg.block_table, pg.page_size, pg.max_blocks_per_seq, pg.page_stride = FAKE.value, ps, 4096, ps * 8 * 128
        s = da.KvScales()
        s.k_scale, s.v_scale = FAKE.value, FAKE.value
        s.stride_b, s.stride_t, s.stride_h = sb, st, 1
        return L.da_gqa_decode_fp8_paged(ctypes.byref(p), ctypes.byref(pg) if pages else None,
                                         ctypes.byref(s) if scales else None, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, FAKE, FAKE, 1 << 40, None)
    assert call(ps=16) == 2                 # fp8 steps are 32 rows
    assert call(st=0) == 2                  # scales varying by page only
    assert call(pages=False) == 1
    assert call(scales=False) == 1
    assert call(p=gqa()) == 1               # not the fp8 dtype
    assert call(ps=24) == 2


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(da, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(da, "_lib", None)
    with pytest.raises(da.LibraryMissing):
        da.lib()


@needs_lib
@cpu_only
def test_noalloc_mla_rejects_oversize_on_the_host():
    # parameters whose workspace exceeds the built-in scratch are rejected
    # before anything else (no device needed, nothing launched)
    L = da.lib()
    assert L.da_noalloc_scratch_bytes() == 64 << 20
    big = mla(512, 128, 32768)
    assert L.da_mla_decode_workspace_size(ctypes.byref(big)) > 64 << 20
    st = L.da_mla_decode_absorbed_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                          None, None)
    assert st == 3
    assert L.da_mla_decode_absorbed_noalloc(ctypes.byref(mla(H=80)), FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                            FAKE, None, None) == 2
    # DeepSeek-V3 MLA at B 64, L 4096 fits
    assert L.da_mla_decode_workspace_size(ctypes.byref(mla())) <= 64 << 20


@cpu_only
def test_host_checks_under_address_and_undefined_behaviour_sanitizers():
    # The argument checks and planners of every entry point, built with
    # AddressSanitizer and UndefinedBehaviorSanitizer on the host side, over a
    # sweep of valid, edge and hostile parameters (the program refuses to run
    # where a GPU could receive its fake pointers).
    import subprocess
    from decode_attention_kv_bf16_amd import build as B
    exe = B.HOST_CHECK_EXE
    srcs = B.sources() + [B.HOST_CHECK_SRC, os.path.join(ROOT, "include", "decode_attn.h")]
    if not os.path.exists(exe) or os.path.getmtime(exe) < max(os.path.getmtime(f) for f in srcs):
        B.build_host_check()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, "5000"], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "host checks passed" in r.stdout


def test_no_kernel_uses_scratch_memory():
    # A kernel that spills vector registers, or keeps a runtime-indexed local
    # array, gets scratch memory; its loads are counted with the untracked
    # load-to-LDS copies, so their waits drain the copy pipelines. The build
    # records the compiler's per-kernel figures; every kernel must have none.
    import json
    from decode_attention_kv_bf16_amd import build as B
    if not os.path.exists(B.RESOURCES_PATH):
        pytest.skip("no build record (run the build first)")
    res = json.load(open(B.RESOURCES_PATH))
    assert len(res) >= 20
    bad = {k: v for k, v in res.items()
           if v.get("ScratchSize [bytes/lane]", 0) or v.get("VGPRs Spill", 0)}
    assert not bad, bad
    for k, v in res.items():
        assert v.get("LDS Size [bytes/block]", 0) <= 160 * 1024, k


@needs_lib
@cpu_only
def test_stream_probes_reject_bad_arguments():
    L = da.lib()
    read, copy = L.da_probe_stream_read, L.da_probe_stream_copy
    big = ctypes.c_void_p(0x40000000)
    assert read(None, 1 << 20, 0, 8, FAKE, None) == 1
    assert read(FAKE, 1 << 20, 0, 8, None, None) == 1
    assert read(FAKE, 0, 0, 8, FAKE, None) == 1
    assert read(FAKE, 24, 0, 8, FAKE, None) == 1            # not a multiple of 16
    assert read(FAKE_MIS, 1 << 20, 0, 8, FAKE, None) == 1
    assert read(FAKE, 1 << 20, -1, 8, FAKE, None) == 1
    assert read(FAKE, 1 << 20, (1 << 20) + 1, 8, FAKE, None) == 1
    for depth in (0, 1, 2, 6, 32):
        assert read(FAKE, 1 << 20, 0, depth, FAKE, None) == 1
        assert copy(FAKE, big, 1 << 20, 0, depth, None) == 1
    assert read(FAKE, 1 << 20, 0, 8, ctypes.c_void_p(FAKE.value + 2), None) == 1
    assert copy(FAKE, None, 1 << 20, 0, 4, None) == 1
    assert copy(FAKE, big, 1 << 20, -5, 4, None) == 1
    assert copy(FAKE, FAKE, 1 << 20, 0, 4, None) == 1        # overlapping
    assert copy(FAKE, ctypes.c_void_p(FAKE.value + 16), 64, 0, 4, None) == 1
    assert copy(FAKE, big, 40, 0, 4, None) == 1
    assert copy(FAKE_MIS, big, 64, 0, 4, None) == 1
