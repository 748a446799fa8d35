"""Float64 reference of decode attention over an FP8 (E4M3) KV cache -- TEST
INFRASTRUCTURE ONLY (imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py; never by the product path).

The page "Attention variants and KV cache" (arganzheng.life, section 6.3,
quantization) stores the cache at one byte per element, FP8 in the E4M3
format (or INT8), halving the bytes per token, with a scale factor per head or
per token (overhead under 1%); at decode the bytes read halve as well. The
page fixes neither the exact scale layout nor the format's bit definition.
Readings used here:
  * E4M3 is the OCP 8-bit floating-point format "E4M3" (1 sign, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal; the
    all-ones exponent with all-ones mantissa is NaN; no infinities; largest
    finite magnitude 448).
  * A cached element's value is decode(code) * scale, with one fp32 scale per
    (sequence, token, KV head) for K and another for V. Scales that are shared
    per head or per token are the same arrays with repeated entries.
The attention itself is then exactly gqa_decode_ref on the decoded values.

Appending into such a cache (the decode step's append, "KV Cache 如何影响了
LLM Inference" section 2.2, with the rotation of oracle/rope.py) quantizes
each new (token, KV head) row x with s = max|x| / 448 (dynamic) or a given s
(static), codes E4M3(x / s) rounded to nearest even, magnitudes clamped to
448. The scale and x / s are taken in float32, the kernel's precision, since
they decide integer codes.

An absorbed-MLA latent cache in E4M3 ("Attention variants and KV cache",
section 4.8 item 3: the nope and rope ranges of a cached row have different
numeric ranges and are quantized apart; section 6.3 for the format and the
halved bytes): row j = [c_kv_j (512) ; k_rope_j (64)] is stored as 576
codes with two fp32 scales per (sequence, token), one for the c_kv range
and one for the k_rope range. Its value is
[decode(codes[:512]) * scale_nope ; decode(codes[512:]) * scale_rope];
the attention is then exactly mla_absorbed_ref on those values. Quantizing
such a row takes each range's own dynamic scale max|range| / 448.

Parity status: pinned by tests/test_oracle_pins.py (decoder against torch's
float8_e4m3fn conversion for all 256 codes and against the format's defining
values; attention against brute force and closed forms with scales; encoder
against the decoder on every finite code, midpoints, clamping and torch's
conversion).
"""
from __future__ import annotations

import numpy as np

from oracle.attention import gqa_decode_ref

E4M3_BIAS = 7
E4M3_MAX = 448.0


def e4m3_to_float(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8 array) as float64, from the format's
    fields: (-1)^s * 2^(e - 7) * (1 + m/8) for e > 0, (-1)^s * 2^-6 * (m/8)
    for e = 0, NaN for e = 15 and m = 7."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - E4M3_BIAS)
    subnormal = (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def dequantize_ref(codes, scales) -> np.ndarray:
    """codes [..., D] uint8 and scales [...] (one per row): decode(code) * scale."""
    return e4m3_to_float(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def gqa_decode_fp8_ref(q, k_codes, v_codes, k_scale, v_scale, seq_lens, scale: float,
                       window: int = 0):
    """GQA decode over an FP8 cache: q [B, Hq, D] float64; k_codes, v_codes
    [B, L, Hkv, D] uint8 E4M3; k_scale, v_scale [B, L, Hkv] (fp32 values).
    Each sequence's first L_b rows are decoded and scaled, then attended as by
    gqa_decode_ref (with its sliding window w, if any). Returns out [B, Hq, D]
    and lse [B, Hq]."""
    seq_lens = np.asarray(seq_lens, np.int64)
    B = q.shape[0]
    L = int(max(1, seq_lens.max(initial=0)))
    k = np.zeros((B, L) + k_codes.shape[2:])
    v = np.zeros((B, L) + v_codes.shape[2:])
    for b in range(B):
        Lb = int(seq_lens[b])
        k[b, :Lb] = dequantize_ref(k_codes[b, :Lb], k_scale[b, :Lb])
        v[b, :Lb] = dequantize_ref(v_codes[b, :Lb], v_scale[b, :Lb])
    return gqa_decode_ref(q, k, v, seq_lens, scale, window)


def e4m3_encode(y) -> np.ndarray:
    """float32 values -> E4M3 codes (uint8), round to nearest even, |y|
    clamped to 448, from the format's fields: below 2^-6 a multiple of 2^-9
    (subnormal), else 1.m with 3 mantissa bits at the value's exponent."""
    y = np.asarray(y, dtype=np.float64)
    sign = np.where(np.signbit(y), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    sub = a < 2.0 ** -6
    m_sub = np.rint(a * 512.0).astype(np.int64)              # numpy rint: half to even
    e = np.floor(np.log2(np.where(sub, 1.0, a))).astype(np.int64)
    q = np.exp2(e - 3.0)
    m = np.rint(np.where(sub, 0.0, a) / q).astype(np.int64)   # 8..16 (16: next binade)
    bump = m == 16
    e = np.where(bump, e + 1, e)
    m = np.where(bump, 8, m)
    normal = ((e + E4M3_BIAS) << 3) | (m - 8)
    return (sign | np.where(sub, m_sub, normal)).astype(np.uint8)


def quantize_rows_ref(x, scale=None):
    """x [..., D] (one row per leading index) -> (codes, scales). Dynamic
    (scale None): s = max|x| / 448 per row; static: the given s per row. In
    float32, as the kernel decides the codes; codes are 0 where s is 0."""
    x32 = np.asarray(x, dtype=np.float32)
    if scale is None:
        s = (np.abs(x32).max(axis=-1) / np.float32(E4M3_MAX)).astype(np.float32)
    else:
        s = np.broadcast_to(np.asarray(scale, np.float32), x32.shape[:-1]).astype(np.float32)
    safe = np.where(s == 0, np.float32(1), s)
    y = (x32 / safe[..., None]).astype(np.float32)
    codes = np.where((s == 0)[..., None], np.uint8(0), e4m3_encode(y))
    return codes.astype(np.uint8), s


def gqa_append_rope_fp8_ref(q, k_new, v_new, positions, max_seq_len: int, rotary_dim: int,
                            style: int, base: float = 10000.0, static_scales=None):
    """The new rows of an append into an E4M3 cache: q and k rotated in fp64
    (oracle.rope.apply_rope_ref), each K and V row quantized by
    quantize_rows_ref. q [B, Hq, D], k_new / v_new [B, Hkv, D] float64;
    static_scales None (dynamic) or a pair of [B, Hkv] arrays. Returns
    (q_rot, k_rot, k_codes, k_scales, v_codes, v_scales, written); the codes
    are those of the rows written at positions[b] for the sequences in
    `written`."""
    from oracle.rope import apply_rope_ref
    positions = np.asarray(positions, np.int64)
    written = (positions >= 0) & (positions < max_seq_len)
    pos = np.where(written, positions, 0)
    q_rot = apply_rope_ref(q, pos, rotary_dim, style, base)
    k_rot = apply_rope_ref(k_new, pos, rotary_dim, style, base)
    ks, vs = (None, None) if static_scales is None else static_scales
    k_codes, k_sc = quantize_rows_ref(k_rot, ks)
    v_codes, v_sc = quantize_rows_ref(np.asarray(v_new, np.float64), vs)
    return q_rot, k_rot, k_codes, k_sc, v_codes, v_sc, written


def gqa_decode_fp8_paged_ref(q, k_pool, v_pool, k_scale_pool, v_scale_pool, block_table,
                             page_size: int, seq_lens, scale: float, window: int = 0):
    """GQA decode over paged E4M3 pools: codes [num_pages, page_size, Hkv, D]
    and scales [num_pages, page_size, Hkv], both addressed through one block
    table ("Attention variants and KV cache" sections 6.1 and 6.3): token t of
    sequence b is row t mod page_size of page block_table[b, t // page_size].
    The attended rows (all, or the last `window`) are gathered in logical
    order, decoded and scaled, then attended as by gqa_decode_ref."""
    from oracle.attention import gqa_decode_ref
    seq_lens = np.asarray(seq_lens, np.int64)
    B = q.shape[0]
    L = int(max(1, seq_lens.max(initial=0)))
    k = np.zeros((B, L) + k_pool.shape[2:])
    v = np.zeros((B, L) + v_pool.shape[2:])
    for b in range(B):
        Lb = int(seq_lens[b])
        lo = max(0, Lb - window) if window > 0 else 0
        for t in range(lo, Lb):
            page, r = int(block_table[b][t // page_size]), t % page_size
            k[b, t] = dequantize_ref(k_pool[page, r], k_scale_pool[page, r])
            v[b, t] = dequantize_ref(v_pool[page, r], v_scale_pool[page, r])
    return gqa_decode_ref(q, k, v, seq_lens, scale, window)


def dequantize_mla_rows_ref(codes, scale_nope, scale_rope, kv_lora_rank: int = 512) -> np.ndarray:
    """Latent rows [..., d_c + d_rope] from E4M3 codes with one scale per row
    for the c_kv range [0, d_c) and one for the k_rope range [d_c, ...)."""
    c = np.asarray(codes, dtype=np.uint8)
    nope = dequantize_ref(c[..., :kv_lora_rank], scale_nope)
    rope = dequantize_ref(c[..., kv_lora_rank:], scale_rope)
    return np.concatenate([nope, rope], axis=-1)


def quantize_mla_rows_ref(rows, kv_lora_rank: int = 512):
    """rows [..., d_c + d_rope] -> (codes, scale_nope, scale_rope): each range
    quantized by quantize_rows_ref with its own dynamic scale."""
    rows = np.asarray(rows)
    cn, sn = quantize_rows_ref(rows[..., :kv_lora_rank])
    cr, sr = quantize_rows_ref(rows[..., kv_lora_rank:])
    return np.concatenate([cn, cr], axis=-1), sn, sr


def mla_absorbed_fp8_ref(q_nope, q_rope, codes, scale_nope, scale_rope, seq_lens, w_uk, w_uv,
                         scale: float, kv_lora_rank: int = 512):
    """Absorbed MLA decode over an E4M3 latent cache: codes [B, L, d_c + d_rope]
    uint8, scale_nope and scale_rope [B, L]; each sequence's first L_b rows are
    dequantized range by range (dequantize_mla_rows_ref) and attended as by
    mla_absorbed_ref. Returns out [B, H, d_v] and lse [B, H]."""
    from oracle.attention import mla_absorbed_ref
    seq_lens = np.asarray(seq_lens, np.int64)
    B = np.shape(q_nope)[0]
    L = int(max(1, seq_lens.max(initial=0)))
    rows = np.zeros((B, L, np.shape(codes)[2]))
    for b in range(B):
        Lb = int(seq_lens[b])
        rows[b, :Lb] = dequantize_mla_rows_ref(codes[b, :Lb], scale_nope[b, :Lb], scale_rope[b, :Lb],
                                               kv_lora_rank)
    return mla_absorbed_ref(q_nope, q_rope, rows, seq_lens, w_uk, w_uv, scale, kv_lora_rank)


def mla_absorbed_fp8_paged_ref(q_nope, q_rope, code_pool, scale_nope_pool, scale_rope_pool, block_table,
                               page_size: int, seq_lens, w_uk, w_uv, scale: float, kv_lora_rank: int = 512):
    """Absorbed MLA decode over a paged E4M3 latent pool ("Attention variants
    and KV cache", section 6.1 for the pages and the block table; sections
    4.8 and 6.3 for the two scaled ranges): code_pool [num_pages, page_size,
    d_c + d_rope] uint8, scale pools [num_pages, page_size] paged like the
    codes. Each sequence's codes and scales are gathered in logical order
    through its table row (oracle.attention.paged_rows_ref), then attended as
    by mla_absorbed_fp8_ref."""
    from oracle.attention import paged_rows_ref
    seq_lens = np.asarray(seq_lens, np.int64)
    B = np.shape(q_nope)[0]
    L = int(max(1, seq_lens.max(initial=0)))
    codes = np.zeros((B, L, np.shape(code_pool)[2]), np.uint8)
    sn = np.zeros((B, L))
    sr = np.zeros((B, L))
    for b in range(B):
        Lb = int(seq_lens[b])
        codes[b, :Lb] = paged_rows_ref(code_pool, block_table[b], page_size, Lb)
        sn[b, :Lb] = paged_rows_ref(scale_nope_pool, block_table[b], page_size, Lb)
        sr[b, :Lb] = paged_rows_ref(scale_rope_pool, block_table[b], page_size, Lb)
    return mla_absorbed_fp8_ref(q_nope, q_rope, codes, sn, sr, seq_lens, w_uk, w_uv, scale, kv_lora_rank)
