"""Float64 reference of the decode step's cache append with rotary position
embedding -- TEST INFRASTRUCTURE ONLY (imported by tests/, __graft_entry__.smoke()
and the CPU-baseline leg of bench.py; never by the product path).

What the pages fix:
  * "KV Cache 如何影响了 LLM Inference" (kakack.github.io), section 2.2: each
    decode step computes one new row of q, k and v for the current token and
    appends the new k and v to the cache, so that the next step finds them
    there; the query is used once and never cached.
  * "Attention variants and KV cache" (arganzheng.life), section 4.2: for MLA
    one projection produces 576 values per token; the first 512 (after an
    RMSNorm, done by the caller) are the latent c_kv, the last 64 are rotated
    and become the decoupled key k^R, which all heads share and which is
    cached after rotation. The rope part of the query is rotated per head.
    Section 4.4: RoPE multiplies a vector at position m by a rotation R_m that
    depends only on m, with R_m^T R_n = R_{n-m}, so a rotated query-key dot
    product depends only on the relative position.
  * "多头潜在注意力（MLA）" (jianzhnie.github.io), section 2: q^R and k^R are
    RoPE applied to their projections.
The pages leave the rotation's form to a later article. Reading used here
(the rotary embedding as commonly defined): the first r entries of a vector
are split into r/2 pairs, and pair i is rotated by the angle m * theta_i with
theta_i = base^(-2i/r) (or caller-given frequencies), counter-clockwise:
    (a, b) -> (a cos(m theta_i) - b sin(m theta_i), a sin(m theta_i) + b cos(m theta_i)).
Entries from r on are left as they are. Two pairings are in use and both are
offered: "half" pairs entry i with entry i + r/2, "interleaved" pairs entries
2i and 2i + 1.

Append semantics: for sequence b with position m = positions[b] in
[0, max_seq_len), the new rows are written at cache row m and the queries are
rotated by m; a position outside that range leaves the sequence alone (no
cache row written, no query written).

Parity status: pinned by tests/test_oracle_rope.py (complex-number form of the
rotation, the relative-position identity of the pages, closed forms at small
sizes, the two pairings related by a permutation, append invariants).
"""
from __future__ import annotations

import numpy as np

STYLE_HALF = 0
STYLE_INTERLEAVED = 1


def rope_inv_freq(rotary_dim: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/r) for i < r/2, in float64."""
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / rotary_dim)


def rope_pairs(rotary_dim: int, style: int):
    """Indices (first, second) of the r/2 rotated pairs."""
    h = rotary_dim // 2
    i = np.arange(h)
    if style == STYLE_HALF:
        return i, i + h
    if style == STYLE_INTERLEAVED:
        return 2 * i, 2 * i + 1
    raise ValueError(f"unknown rope style {style}")


def apply_rope_ref(x, positions, rotary_dim: int, style: int, base: float = 10000.0,
                   inv_freq=None) -> np.ndarray:
    """Rotate x [B, ..., n] (float64) by the position of its sequence,
    positions [B]. Returns a new float64 array."""
    x = np.array(x, dtype=np.float64, copy=True)
    theta = rope_inv_freq(rotary_dim, base) if inv_freq is None else np.asarray(inv_freq, np.float64)
    a_idx, b_idx = rope_pairs(rotary_dim, style)
    pos = np.asarray(positions, dtype=np.float64)
    for bi in range(x.shape[0]):
        phi = pos[bi] * theta                       # [r/2]
        c, s = np.cos(phi), np.sin(phi)
        a = x[bi][..., a_idx].copy()
        b = x[bi][..., b_idx].copy()
        x[bi][..., a_idx] = a * c - b * s
        x[bi][..., b_idx] = a * s + b * c
    return x


def cache_row_index(b: int, t: int, block_table=None, page_size: int = 0):
    """(first index, row) of token t of sequence b: (b, t) for a contiguous
    cache, (page, t mod page_size) for a paged pool, where page is the table
    entry of block t // page_size."""
    if block_table is None:
        return b, t
    return int(block_table[b, t // page_size]), t % page_size


def gqa_append_rope_ref(q, k_new, v_new, positions, k_cache, v_cache, max_seq_len: int,
                        rotary_dim: int, style: int, base: float = 10000.0, inv_freq=None,
                        block_table=None, page_size: int = 0):
    """q [B, Hq, D], k_new and v_new [B, Hkv, D]; k_cache, v_cache
    [B, L, Hkv, D] or paged pools [pages, page_size, Hkv, D]. Returns
    (q_out, k_cache', v_cache', written) with float64 copies: q_out holds the
    rotated queries (NaN rows for skipped sequences), the caches the new rows,
    `written` [B] bool which sequences were appended."""
    q = np.asarray(q, np.float64)
    k_cache = np.array(k_cache, dtype=np.float64, copy=True)
    v_cache = np.array(v_cache, dtype=np.float64, copy=True)
    positions = np.asarray(positions, np.int64)
    written = (positions >= 0) & (positions < max_seq_len)
    pos_rot = np.where(written, positions, 0)
    q_rot = apply_rope_ref(q, pos_rot, rotary_dim, style, base, inv_freq)
    k_rot = apply_rope_ref(k_new, pos_rot, rotary_dim, style, base, inv_freq)
    q_out = np.full_like(q_rot, np.nan)
    for b in range(q.shape[0]):
        if not written[b]:
            continue
        q_out[b] = q_rot[b]
        i, t = cache_row_index(b, int(positions[b]), block_table, page_size)
        k_cache[i, t] = k_rot[b]
        v_cache[i, t] = np.asarray(v_new[b], np.float64)
    return q_out, k_cache, v_cache, written


def mla_append_rope_ref(q_rope, kv_new, positions, cache, max_seq_len: int, rotary_dim: int,
                        style: int, base: float = 10000.0, inv_freq=None, block_table=None,
                        page_size: int = 0, d_c: int = 512):
    """q_rope [B, H, d_rope]; kv_new [B, d_c + d_rope] = [c_kv ; k_rope before
    rotation]; cache [B, L, d_c + d_rope] or a paged pool [pages, page_size,
    d_c + d_rope]. The cached row is [c_kv ; RoPE(k_rope)]. Returns (q_rope_out,
    cache', written) as gqa_append_rope_ref."""
    q_rope = np.asarray(q_rope, np.float64)
    kv_new = np.asarray(kv_new, np.float64)
    cache = np.array(cache, dtype=np.float64, copy=True)
    positions = np.asarray(positions, np.int64)
    written = (positions >= 0) & (positions < max_seq_len)
    pos_rot = np.where(written, positions, 0)
    q_rot = apply_rope_ref(q_rope, pos_rot, rotary_dim, style, base, inv_freq)
    k_rot = apply_rope_ref(kv_new[:, d_c:], pos_rot, rotary_dim, style, base, inv_freq)
    q_out = np.full_like(q_rot, np.nan)
    for b in range(q_rope.shape[0]):
        if not written[b]:
            continue
        q_out[b] = q_rot[b]
        i, t = cache_row_index(b, int(positions[b]), block_table, page_size)
        cache[i, t, :d_c] = kv_new[b, :d_c]
        cache[i, t, d_c:] = k_rot[b]
    return q_out, cache, written
