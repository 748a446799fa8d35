"""Seeded synthetic inputs for single-token decode attention over a KV cache.

This module holds no attention arithmetic: it only draws random numbers,
rounds them to bfloat16 and lays them out. Both the CPU oracle tests and the
GPU path take their inputs from here, so both see identical bits.

Shapes follow the models the pages analyse:
  * Llama-3-8B GQA (32 query heads / 8 KV heads, d_head 128) -- "Attention
    variants and KV cache" (arganzheng.life), section 1.1 model baseline;
  * Llama-2-7B MHA (32 heads, d_head 128) -- AIFAQ page, per-token element
    counts for LlaMA-2-7B; kakack.github.io KV-cache page, section 5;
  * DeepSeek-V3 MLA (128 heads, kv_lora_rank 512, rope 64, nope 128, v 128)
    -- arganzheng.life section 4.2 config.json; jianzhnie.github.io MLA page,
    section 3 (actual parameter configuration).

Seeding recipe (every stream is numpy PCG64 via ``default_rng``):
  * per-sequence lengths:       default_rng([seed, cfg, 0]) .integers(lo, hi, endpoint=True)
  * queries (q, or q_nope then q_rope): default_rng([seed, cfg, 1])
  * cache of sequence b (K then V, or latent rows [c_kv | k_rope]):
                                default_rng([seed, cfg, 2, b])
  * W_UK:                       default_rng([seed, cfg, 3])
  * W_UV:                       default_rng([seed, cfg, 4])
  * append positions:           default_rng([seed, cfg, 5]) .integers(0, L_max)
  * appended rows (q, k_new, v_new; or q_rope, kv_new): default_rng([seed, cfg, 6])
Normals are drawn in float32 and rounded to bfloat16 with round-to-nearest-even.
W_UK / W_UV are N(0, 1/512): variance 1/512, i.e. standard deviation 1/sqrt(512).

A padded cache has layout [B, L_max, H_kv, D] (GQA) or [B, L_max, 576] (MLA);
rows at or past a sequence's length are filled with ``pad_value`` (NaN in
parity runs, so that any read past the end of a sequence poisons the output).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

BASE_SEED = 0

BF16_NAN_BITS = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# bfloat16 helpers (storage only: bf16 values are kept as uint16 bit patterns)
# ----------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    Inputs here are finite normals, so no NaN special-casing is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exactly equal float32 values."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class GQAShape:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    # either a fixed length for every sequence, or an inclusive uniform range
    seq_len: Optional[int] = None
    seq_len_range: Optional[tuple] = None
    dtype: str = "bf16"  # "bf16" or "f32"
    name: str = "gqa"


@dataclass(frozen=True)
class MLAShape:
    batch: int
    num_heads: int = 128
    seq_len: Optional[int] = None
    seq_len_range: Optional[tuple] = None
    kv_lora_rank: int = 512
    qk_rope_dim: int = 64
    qk_nope_dim: int = 128
    v_head_dim: int = 128
    name: str = "mla"


# The five workloads: a tiny fp32 GQA case, Llama-3-8B GQA, DeepSeek-V3 MLA,
# long-context MLA and ragged Llama-2-7B-shaped MHA.
CONFIGS = {
    1: GQAShape(1, 4, 2, 64, seq_len=128, dtype="f32", name="gqa-tiny-f32-b1-h4-kv2-d64-l128"),
    2: GQAShape(32, 32, 8, 128, seq_len=4096, name="llama3-8b-gqa-b32-l4096"),
    3: MLAShape(64, 128, seq_len=4096, name="deepseek-v3-mla-b64-l4096"),
    4: MLAShape(4, 128, seq_len_range=(16384, 32768), name="deepseek-v3-mla-longctx-b4-l16k-32k"),
    5: GQAShape(64, 32, 32, 128, seq_len_range=(1, 8192), name="llama2-7b-mha-ragged-b64-l1-8192"),
}


def draw_seq_lens(batch: int, seq_len=None, seq_len_range=None, cfg: int = 0,
                  seed: int = BASE_SEED) -> np.ndarray:
    if seq_len is not None:
        return np.full(batch, int(seq_len), dtype=np.int32)
    lo, hi = seq_len_range
    rng = np.random.default_rng([seed, cfg, 0])
    return rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


# ----------------------------------------------------------------------------
# GQA / MQA / MHA
# ----------------------------------------------------------------------------

@dataclass
class GQAInputs:
    """Host copies of one GQA decode problem.

    q: [B, Hq, D]; k, v: [B, L_max, Hkv, D]. For dtype "bf16" arrays hold
    uint16 bit patterns, for "f32" they hold float32 values.
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    seq_lens: np.ndarray
    dtype: str
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, Hq, D = self.q.shape
        return B, Hq, self.k.shape[2], D, self.k.shape[1]

    def as_f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def _store(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x_f32) if dtype == "bf16" else np.ascontiguousarray(x_f32, np.float32)


def _pad_fill(dtype: str, pad_value: float):
    if dtype == "bf16":
        if np.isnan(pad_value):
            return BF16_NAN_BITS
        return bf16_round(np.array([pad_value], np.float32))[0]
    return np.float32(pad_value)


def make_gqa(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
             seq_lens: Sequence[int], dtype: str = "bf16", cfg: int = 0,
             seed: int = BASE_SEED, max_seq_len: Optional[int] = None,
             pad_value: float = 0.0, only_seqs: Optional[Sequence[int]] = None) -> GQAInputs:
    """Draw q, K, V ~ N(0, 1) for a GQA decode step.

    ``only_seqs`` restricts cache generation to the listed sequences (other
    sequences stay filled with ``pad_value``); their bits are identical to a
    full generation because each sequence owns its own random stream.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (batch,)
    L_max = int(max_seq_len if max_seq_len is not None else max(1, int(seq_lens.max(initial=0))))
    assert int(seq_lens.max(initial=0)) <= L_max
    B, Hq, Hkv, D = batch, num_q_heads, num_kv_heads, head_dim
    rq = np.random.default_rng([seed, cfg, 1])
    q = _store(_normal(rq, (B, Hq, D)), dtype)
    store_dt = np.uint16 if dtype == "bf16" else np.float32
    k = np.empty((B, L_max, Hkv, D), dtype=store_dt)
    v = np.empty((B, L_max, Hkv, D), dtype=store_dt)
    fill = _pad_fill(dtype, pad_value)

    def one(b):
        L = int(seq_lens[b])
        k[b, L:] = fill
        v[b, L:] = fill
        if only_seqs is not None and b not in only_seqs:
            k[b, :L] = fill
            v[b, :L] = fill
            return
        r = np.random.default_rng([seed, cfg, 2, b])
        k[b, :L] = _store(_normal(r, (L, Hkv, D)), dtype)
        v[b, :L] = _store(_normal(r, (L, Hkv, D)), dtype)

    if B > 1 and int(seq_lens.sum()) * Hkv * D > (1 << 22):
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(B)))
    else:
        for b in range(B):
            one(b)
    scale = 1.0 / float(np.sqrt(D))
    return GQAInputs(q, k, v, seq_lens, dtype, scale,
                     meta=dict(cfg=cfg, seed=seed, pad_value=pad_value))


def make_gqa_config(cfg: int, seed: int = BASE_SEED, pad_value: float = 0.0,
                    only_seqs=None, batch: Optional[int] = None) -> GQAInputs:
    s = CONFIGS[cfg]
    assert isinstance(s, GQAShape)
    B = s.batch if batch is None else batch
    lens = draw_seq_lens(s.batch, s.seq_len, s.seq_len_range, cfg, seed)[:B]
    L_max = s.seq_len if s.seq_len is not None else s.seq_len_range[1]
    return make_gqa(B, s.num_q_heads, s.num_kv_heads, s.head_dim, lens, s.dtype,
                    cfg=cfg, seed=seed, max_seq_len=L_max, pad_value=pad_value,
                    only_seqs=only_seqs)


# ----------------------------------------------------------------------------
# absorbed MLA
# ----------------------------------------------------------------------------

@dataclass
class MLAInputs:
    """Host copies (bf16 bit patterns) of one absorbed-MLA decode problem.

    q_nope [B,H,d_nope], q_rope [B,H,d_rope], cache [B,L_max,d_c+d_rope]
    (row = [c_kv | k_rope]), w_uk and w_uv [H, d_c, d_nope] / [H, d_c, d_v].
    """
    q_nope: np.ndarray
    q_rope: np.ndarray
    cache: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    seq_lens: np.ndarray
    scale: float
    meta: dict = field(default_factory=dict)

    def as_f64(self, name: str) -> np.ndarray:
        return bf16_to_f32(getattr(self, name)).astype(np.float64)


def make_mla(batch: int, num_heads: int, seq_lens: Sequence[int], cfg: int = 0,
             seed: int = BASE_SEED, max_seq_len: Optional[int] = None,
             kv_lora_rank: int = 512, qk_rope_dim: int = 64, qk_nope_dim: int = 128,
             v_head_dim: int = 128, pad_value: float = 0.0,
             only_seqs: Optional[Sequence[int]] = None) -> MLAInputs:
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (batch,)
    L_max = int(max_seq_len if max_seq_len is not None else max(1, int(seq_lens.max(initial=0))))
    B, H = batch, num_heads
    row = kv_lora_rank + qk_rope_dim
    rq = np.random.default_rng([seed, cfg, 1])
    q_nope = bf16_round(_normal(rq, (B, H, qk_nope_dim)))
    q_rope = bf16_round(_normal(rq, (B, H, qk_rope_dim)))
    cache = np.empty((B, L_max, row), dtype=np.uint16)
    fill = _pad_fill("bf16", pad_value)

    def one(b):
        L = int(seq_lens[b])
        cache[b, L:] = fill
        if only_seqs is not None and b not in only_seqs:
            cache[b, :L] = fill
            return
        r = np.random.default_rng([seed, cfg, 2, b])
        cache[b, :L] = bf16_round(_normal(r, (L, row)))

    if B > 1 and int(seq_lens.sum()) * row > (1 << 22):
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(B)))
    else:
        for b in range(B):
            one(b)
    std = 1.0 / float(np.sqrt(kv_lora_rank))
    w_uk = bf16_round(_normal(np.random.default_rng([seed, cfg, 3]), (H, kv_lora_rank, qk_nope_dim), std))
    w_uv = bf16_round(_normal(np.random.default_rng([seed, cfg, 4]), (H, kv_lora_rank, v_head_dim), std))
    scale = 1.0 / float(np.sqrt(qk_nope_dim + qk_rope_dim))
    return MLAInputs(q_nope, q_rope, cache, w_uk, w_uv, seq_lens, scale,
                     meta=dict(cfg=cfg, seed=seed, pad_value=pad_value))


def make_mla_config(cfg: int, seed: int = BASE_SEED, pad_value: float = 0.0,
                    only_seqs=None, batch: Optional[int] = None) -> MLAInputs:
    s = CONFIGS[cfg]
    assert isinstance(s, MLAShape)
    B = s.batch if batch is None else batch
    lens = draw_seq_lens(s.batch, s.seq_len, s.seq_len_range, cfg, seed)[:B]
    L_max = s.seq_len if s.seq_len is not None else s.seq_len_range[1]
    return make_mla(B, s.num_heads, lens, cfg=cfg, seed=seed, max_seq_len=L_max,
                    kv_lora_rank=s.kv_lora_rank, qk_rope_dim=s.qk_rope_dim,
                    qk_nope_dim=s.qk_nope_dim, v_head_dim=s.v_head_dim,
                    pad_value=pad_value, only_seqs=only_seqs)


@dataclass
class MLAFp8Inputs:
    """Host copies of one absorbed-MLA decode problem over an E4M3 latent cache.

    q_nope, q_rope, w_uk, w_uv as in MLAInputs (bf16 bit patterns); cache
    [B, L_max, d_c + d_rope] uint8 E4M3 codes; scale_nope, scale_rope
    [B, L_max] float32: row (b, t) stands for
    [code[:d_c] * scale_nope[b, t] ; code[d_c:] * scale_rope[b, t]].
    """
    q_nope: np.ndarray
    q_rope: np.ndarray
    cache: np.ndarray
    scale_nope: np.ndarray
    scale_rope: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    seq_lens: np.ndarray
    scale: float
    meta: dict = field(default_factory=dict)


def make_mla_fp8(batch: int, num_heads: int, seq_lens: Sequence[int], cfg: int = 0,
                 seed: int = BASE_SEED, max_seq_len: Optional[int] = None,
                 rope_std: float = 1.0, pad_nan: bool = True) -> MLAFp8Inputs:
    """DeepSeek-V3 latent shapes (d_c 512, d_rope 64, d_nope = d_v = 128). The
    queries and weights are make_mla's (same streams); each cached row is drawn
    as make_mla draws it (k_rope times rope_std), in float32, and each of its
    two ranges is quantized with its own scale max|range| / 448. Rows past a
    sequence's length hold the NaN code and NaN scales when pad_nan, else 0."""
    m = make_mla(batch, num_heads, [0] * batch, cfg=cfg, seed=seed, max_seq_len=1)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    L_max = int(max_seq_len if max_seq_len is not None else max(1, int(seq_lens.max(initial=0))))
    B = batch
    codes = np.full((B, L_max, 576), FP8_NAN_CODE if pad_nan else 0, np.uint8)
    pad = np.float32(np.nan if pad_nan else 0.0)
    sn = np.full((B, L_max), pad, np.float32)
    sr = np.full((B, L_max), pad, np.float32)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        x = _normal(np.random.default_rng([seed, cfg, 2, b]), (L, 576))
        x[:, 512:] *= np.float32(rope_std)
        for lo, hi, sc in ((0, 512, sn), (512, 576, sr)):
            s = (np.maximum(np.abs(x[:, lo:hi]).max(axis=1), 1e-30) / E4M3_MAX).astype(np.float32)
            codes[b, :L, lo:hi] = encode_e4m3(x[:, lo:hi] / s[:, None])
            sc[b, :L] = s
    return MLAFp8Inputs(m.q_nope, m.q_rope, codes, sn, sr, m.w_uk, m.w_uv, seq_lens, m.scale,
                        meta=dict(cfg=cfg, seed=seed, rope_std=rope_std))


def make_mla_fp8_config(cfg: int, seed: int = BASE_SEED) -> MLAFp8Inputs:
    """An MLA config's shapes and lengths with the latent cache in E4M3."""
    s = CONFIGS[cfg]
    assert isinstance(s, MLAShape)
    lens = draw_seq_lens(s.batch, s.seq_len, s.seq_len_range, cfg, seed)
    L_max = s.seq_len if s.seq_len is not None else s.seq_len_range[1]
    return make_mla_fp8(s.batch, s.num_heads, lens, cfg=cfg, seed=seed, max_seq_len=L_max)


# ----------------------------------------------------------------------------
# paged caches
# ----------------------------------------------------------------------------

def make_block_table(seq_lens: Sequence[int], page_size: int, seed: int = BASE_SEED,
                     spare_pages: int = 3, max_blocks: Optional[int] = None):
    """A block table for a paged cache: sequence b owns ceil(L_b / page_size)
    pages, placed at seeded random physical positions of a pool that also
    holds ``spare_pages`` unused pages. Entries past a sequence's pages are -1.
    Returns (table [B, max_blocks] int32, number of pages in the pool)."""
    seq_lens = np.asarray(seq_lens, np.int64)
    n_blocks = -(-seq_lens // page_size)
    width = int(max_blocks if max_blocks is not None else max(1, n_blocks.max(initial=0)))
    assert width >= n_blocks.max(initial=0)
    num_pages = int(n_blocks.sum()) + spare_pages
    perm = np.random.default_rng([seed, 77]).permutation(num_pages)
    table = np.full((len(seq_lens), width), -1, np.int32)
    k = 0
    for b, nb in enumerate(n_blocks):
        table[b, :nb] = perm[k:k + nb]
        k += int(nb)
    return table, num_pages


def paginate(cache: np.ndarray, seq_lens: Sequence[int], table: np.ndarray, num_pages: int,
             page_size: int, fill) -> np.ndarray:
    """Copy rows [0, L_b) of each sequence of a contiguous cache [B, L, ...]
    into a pool [num_pages, page_size, ...] as the block table says; every
    other pool row (spare pages, the tail of a last page) holds ``fill``."""
    pool = np.full((num_pages, page_size) + cache.shape[2:], fill, dtype=cache.dtype)
    for b, L in enumerate(np.asarray(seq_lens, np.int64)):
        for j in range(-(-int(L) // page_size)):
            rows = cache[b, j * page_size:min((j + 1) * page_size, int(L))]
            pool[int(table[b, j]), :len(rows)] = rows
    return pool


# ----------------------------------------------------------------------------
# FP8 (E4M3) caches ("Attention variants and KV cache", section 6.3)
# ----------------------------------------------------------------------------

FP8_NAN_CODE = np.uint8(0x7F)
E4M3_MAX = 448.0


@dataclass
class GQAFp8Inputs:
    """Host copies of one GQA decode problem over an FP8 cache.

    q [B, Hq, D] bf16 bit patterns; k, v [B, L_max, H_kv, D] uint8 E4M3 codes;
    k_scale, v_scale [B, L_max, H_kv] float32: element (b, t, h, :) of K stands
    for code * k_scale[b, t, h].
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    k_scale: np.ndarray
    v_scale: np.ndarray
    seq_lens: np.ndarray
    scale: float
    meta: dict = field(default_factory=dict)


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 values (|x| <= 448) -> E4M3 codes, round to nearest even, by
    torch's float8_e4m3fn conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def make_gqa_fp8(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 seq_lens: Sequence[int], cfg: int = 0, seed: int = BASE_SEED,
                 max_seq_len: Optional[int] = None, scales: str = "token",
                 pad_nan: bool = True) -> GQAFp8Inputs:
    """q, K, V ~ N(0, 1) drawn from the same streams as make_gqa, with K and V
    quantized to E4M3. scales="token": one scale per (sequence, token, KV
    head) row, amax(|row|) / 448; scales="head": one per KV head over the whole
    batch (repeated in the arrays). Rows past a sequence's length hold the NaN
    code and NaN scales when pad_nan, else zeros."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (batch,)
    L_max = int(max_seq_len if max_seq_len is not None else max(1, int(seq_lens.max(initial=0))))
    assert int(seq_lens.max(initial=0)) <= L_max
    B, Hq, Hkv, D = batch, num_q_heads, num_kv_heads, head_dim
    q = bf16_round(_normal(np.random.default_rng([seed, cfg, 1]), (B, Hq, D)))
    kf = np.zeros((B, L_max, Hkv, D), np.float32)
    vf = np.zeros((B, L_max, Hkv, D), np.float32)
    for b in range(B):
        L = int(seq_lens[b])
        r = np.random.default_rng([seed, cfg, 2, b])
        kf[b, :L] = _normal(r, (L, Hkv, D))
        vf[b, :L] = _normal(r, (L, Hkv, D))
    valid = np.arange(L_max)[None, :] < seq_lens[:, None]          # [B, L]
    out = []
    for x in (kf, vf):
        amax = np.abs(x).max(axis=-1)                                # [B, L, Hkv]
        if scales == "head":
            amax = np.broadcast_to(np.where(valid[..., None], amax, 0).max(axis=(0, 1)), amax.shape)
        elif scales != "token":
            raise ValueError(scales)
        s = (np.maximum(amax, 1e-30) / E4M3_MAX).astype(np.float32)
        codes = encode_e4m3(x / s[..., None])
        pad_code, pad_scale = (FP8_NAN_CODE, np.nan) if pad_nan else (0, 0.0)
        codes[~valid] = pad_code
        s = np.where(valid[..., None], s, np.float32(pad_scale)).astype(np.float32)
        out += [codes, s]
    k, ks, v, vs = out
    return GQAFp8Inputs(q, k, v, ks, vs, seq_lens, 1.0 / float(np.sqrt(D)),
                        meta=dict(cfg=cfg, seed=seed, scales=scales))


def make_gqa_fp8_config(cfg: int, seed: int = BASE_SEED, scales: str = "token",
                        pad_nan: bool = False, batch: Optional[int] = None) -> GQAFp8Inputs:
    """The shapes and lengths of a GQA config with the cache in E4M3."""
    s = CONFIGS[cfg]
    assert isinstance(s, GQAShape)
    B = s.batch if batch is None else batch
    lens = draw_seq_lens(s.batch, s.seq_len, s.seq_len_range, cfg, seed)[:B]
    L_max = s.seq_len if s.seq_len is not None else s.seq_len_range[1]
    return make_gqa_fp8(B, s.num_q_heads, s.num_kv_heads, s.head_dim, lens, cfg=cfg, seed=seed,
                        max_seq_len=L_max, scales=scales, pad_nan=pad_nan)


# ----------------------------------------------------------------------------
# cache append: the new token's rows
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class AppendInputs:
    """The new rows of one decode step. GQA: q [B, Hq, D] and k_new, v_new
    [B, Hkv, D]; MLA: q [B, H, 64] (the rope part of the queries), k_new
    [B, 576] ([c_kv | k_rope] before rotation) and v_new None. positions [B]
    int32. Storage as GQAInputs (uint16 bit patterns for bf16)."""
    q: np.ndarray
    k_new: np.ndarray
    v_new: Optional[np.ndarray]
    positions: np.ndarray
    dtype: str

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return (bf16_to_f32(a) if self.dtype == "bf16" else a).astype(np.float64)


def draw_positions(batch: int, max_seq_len: int, cfg: int = 0, seed: int = BASE_SEED) -> np.ndarray:
    rng = np.random.default_rng([seed, cfg, 5])
    return rng.integers(0, max_seq_len, size=batch).astype(np.int32)


def make_gqa_append(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    max_seq_len: int, dtype: str = "bf16", cfg: int = 0, seed: int = BASE_SEED,
                    positions: Optional[Sequence[int]] = None) -> AppendInputs:
    rng = np.random.default_rng([seed, cfg, 6])
    q = _store(_normal(rng, (batch, num_q_heads, head_dim)), dtype)
    k = _store(_normal(rng, (batch, num_kv_heads, head_dim)), dtype)
    v = _store(_normal(rng, (batch, num_kv_heads, head_dim)), dtype)
    pos = draw_positions(batch, max_seq_len, cfg, seed) if positions is None else \
        np.asarray(positions, np.int32)
    return AppendInputs(q, k, v, pos, dtype)


def make_mla_append(batch: int, num_heads: int, max_seq_len: int, cfg: int = 0,
                    seed: int = BASE_SEED, positions: Optional[Sequence[int]] = None,
                    d_c: int = 512, d_rope: int = 64) -> AppendInputs:
    rng = np.random.default_rng([seed, cfg, 6])
    q_rope = bf16_round(_normal(rng, (batch, num_heads, d_rope)))
    kv_new = bf16_round(_normal(rng, (batch, d_c + d_rope)))
    pos = draw_positions(batch, max_seq_len, cfg, seed) if positions is None else \
        np.asarray(positions, np.int32)
    return AppendInputs(q_rope, kv_new, None, pos, "bf16")
