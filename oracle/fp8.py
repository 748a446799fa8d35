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

Parity status: pinned by tests/test_oracle_pins.py (decoder against torch's
float8_e4m3fn conversion for all 256 codes and against the format's defining
values; attention against brute force and closed forms with scales).
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
