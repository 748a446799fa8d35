"""Float64 reference definitions of decode attention -- TEST INFRASTRUCTURE ONLY.

Every function works on float64 numpy arrays holding the exact values the GPU
receives (bfloat16 inputs are widened exactly before they get here), one
sequence at a time, with no blocking, fusion or reordering beyond what the
definitions state. A library primitive (numpy matmul / exp / log) is used for
each step.

Conventions (readings of the pages where they are silent):
  * exp base: natural; lse = log(sum_j exp(s_j)), evaluated as m + log(sum exp(s - m)).
  * a sequence of length 0 attends nothing: out = 0, lse = -inf (the identity
    element of the split-KV merge).
  * no causal mask at decode: the new token's K/V are already in the cache and
    every one of the L_b cached rows is attended.

Parity status: every function here is pinned by tests against closed forms,
brute force on tiny inputs, associativity, or torch's scaled_dot_product_attention.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _softmax_attend(scores: np.ndarray, values: np.ndarray):
    """Softmax over the token axis of ``scores`` and the weighted sum of ``values``.

    scores: [L, H] (token, head); values: [L, H, Dv] or [L, Dv] (shared by all heads).
    Returns out [H, Dv] and lse [H].

    Standard softmax attention as written in the kakack.github.io KV-cache
    page (section 4, UnifiedAttention forward: softmax of the scaled scores
    times V) and the arganzheng.life page, section 2.1 (per-head attention).
    """
    L = scores.shape[0]
    H = scores.shape[1]
    Dv = values.shape[-1]
    if L == 0:
        return np.zeros((H, Dv)), np.full(H, NEG_INF)
    m = scores.max(axis=0)                      # [H]
    w = np.exp(scores - m[None, :])             # [L, H]
    z = w.sum(axis=0)                           # [H]
    lse = m + np.log(z)
    p = w / z[None, :]                          # softmax weights, rows sum to 1
    if values.ndim == 2:                        # one value row per token, shared by all heads
        out = p.T @ values                      # [H, Dv]
    else:                                       # [L, H, Dv]
        out = np.einsum("lh,lhd->hd", p, values)
    return out, lse


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``h``: contiguous groups of g = Hq/Hkv heads.

    Query heads [k*g, (k+1)*g) share KV head k (kakack.github.io page,
    section 4, the 8-query / 2-KV example; arganzheng.life section 3.2 diagram;
    shippingwang.com chapter 7, section 7.3: the kernel maps q_head // g).
    """
    g = num_q_heads // num_kv_heads
    return h // g


def gqa_decode_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens, scale: float,
                   window: int = 0):
    """GQA / MQA / MHA decode for one new query token per sequence.

    q [B, Hq, D]; k, v [B, L_max, Hkv, D] (cache layout [B, L, n_kv, d_head]);
    seq_lens [B]; scale usually 1/sqrt(D).
    Returns out [B, Hq, D] and lse [B, Hq] (natural log).

    window w > 0: sliding-window attention, only the last w rows
    [max(0, L - w), L) are attended ("Attention variants and KV cache",
    section 5.3: each query sees at most w keys, the cache need keep only
    the latest w tokens). w = 0 attends all L rows.

    s_j = scale * q_h . k_{j, kv(h)};  p = softmax_j(s);  o_h = sum_j p_j v_{j, kv(h)}.
    Decode reads the whole cache once per step (arganzheng.life section 2.2;
    kakack.github.io section 2.2); GQA semantics from arganzheng.life
    section 3.2 and the kakack.github.io UnifiedAttention module (section 4),
    whose assert requires Hq % Hkv == 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("number of query heads must be a multiple of the number of KV heads")
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), NEG_INF)
    kv_of = np.array([kv_head_of(h, Hq, Hkv) for h in range(Hq)])
    for b in range(B):
        L = int(seq_lens[b])
        lo = max(0, L - window) if window > 0 else 0
        Kb = k[b, lo:L][:, kv_of, :]            # [rows, Hq, D]: the KV row each query head reads
        Vb = v[b, lo:L][:, kv_of, :]
        s = scale * np.einsum("lhd,hd->lh", Kb, q[b])
        out[b], lse[b] = _softmax_attend(s, Vb)
    return out, lse


def absorb_query_ref(q_nope: np.ndarray, w_uk: np.ndarray):
    """Query-side absorption: q~_h = q_nope_h . W_UK,h^T (per head, 512-d latent).

    q_nope [B, H, d_nope]; w_uk [H, d_c, d_nope] is the per-head slice of the
    row-vector up-projection, k^C_{j,h} = c_j W_UK[h], i.e.
    k^C_{j,h}[e] = sum_c c_j[c] W_UK[h, c, e] (jianzhnie.github.io section 2).
    Returns q~ [B, H, d_c] with q~[b,h,c] = sum_e W_UK[h,c,e] q_nope[b,h,e],
    so that q~_h . c_j = q_nope_h . k^C_{j,h}.

    Matrix absorption by re-association: arganzheng.life section 4.5 (query
    side) and jianzhnie.github.io MLA page, section 4 (the "Absorb" line).
    """
    return np.einsum("hce,bhe->bhc", np.asarray(w_uk, np.float64), np.asarray(q_nope, np.float64))


def mla_absorbed_ref(q_nope, q_rope, cache, seq_lens, w_uk, w_uv, scale: float,
                     kv_lora_rank: int = 512):
    """DeepSeek-style MLA decode with matrix absorption.

    q_nope [B,H,d_nope], q_rope [B,H,d_rope], cache [B,L_max,d_c+d_rope] with
    row j = [c_kv_j (d_c) ; k_rope_j (d_rope)] shared by every head,
    w_uk [H,d_c,d_nope], w_uv [H,d_c,d_v]; scale = 1/sqrt(d_nope + d_rope).
    Returns out [B,H,d_v] and lse [B,H].

    Steps (arganzheng.life section 4.5; jianzhnie.github.io section 4):
      1. q~_h = q_nope_h W_UK,h^T                          (512-d)
      2. q^_h = [q~_h ; q_rope_h]                           (576-d)
      3. s_j = scale * q^_h . cache_j                       (one 576-d dot per row)
      4. p = softmax_j(s)
      5. o~_h = sum_j p_j c_kv_j   (V is the first d_c columns of the same row)
      6. o_h = o~_h W_UV,h
    The scale stays 1/sqrt(192), not 1/sqrt(576) (arganzheng.life section 4.5).
    """
    q_nope = np.asarray(q_nope, np.float64)
    q_rope = np.asarray(q_rope, np.float64)
    cache = np.asarray(cache, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    B, H, _ = q_nope.shape
    d_c = kv_lora_rank
    d_v = w_uv.shape[2]
    q_tilde = absorb_query_ref(q_nope, w_uk)                    # [B, H, d_c]
    q_hat = np.concatenate([q_tilde, q_rope], axis=2)           # [B, H, d_c + d_rope]
    out = np.zeros((B, H, d_v))
    lse = np.full((B, H), NEG_INF)
    for b in range(B):
        L = int(seq_lens[b])
        C = cache[b, :L]                                        # [L, 576]
        s = scale * (C @ q_hat[b].T)                            # [L, H]
        o_lat, lse[b] = _softmax_attend(s, C[:, :d_c])          # [H, d_c]
        out[b] = np.einsum("hc,hce->he", o_lat, w_uv)
    return out, lse


def mla_explicit_ref(q_nope, q_rope, cache, seq_lens, w_uk, w_uv, scale: float,
                     kv_lora_rank: int = 512):
    """MLA decode by the literal formula: up-project every cached latent.

    k_{j,h} = [c_kv_j W_UK,h ; k_rope_j] (d_nope + d_rope), v_{j,h} = c_kv_j W_UV,h,
    q_h = [q_nope_h ; q_rope_h], then standard softmax attention with
    scale 1/sqrt(d_nope + d_rope).
    jianzhnie.github.io MLA page, section 2 (KV computation, output o_{t,i})
    and section 4 (the "Normal" line); arganzheng.life section 4.2.
    """
    q_nope = np.asarray(q_nope, np.float64)
    q_rope = np.asarray(q_rope, np.float64)
    cache = np.asarray(cache, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    B, H, _ = q_nope.shape
    d_c = kv_lora_rank
    d_v = w_uv.shape[2]
    out = np.zeros((B, H, d_v))
    lse = np.full((B, H), NEG_INF)
    q_full = np.concatenate([q_nope, q_rope], axis=2)           # [B, H, 192]
    for b in range(B):
        L = int(seq_lens[b])
        c_kv = cache[b, :L, :d_c]                               # [L, d_c]
        k_rope = cache[b, :L, d_c:]                             # [L, d_rope]
        k_content = np.einsum("lc,hce->lhe", c_kv, w_uk)        # [L, H, d_nope]
        k_full = np.concatenate(
            [k_content, np.broadcast_to(k_rope[:, None, :], (L, H, k_rope.shape[1]))], axis=2)
        v_full = np.einsum("lc,hce->lhe", c_kv, w_uv)           # [L, H, d_v]
        s = scale * np.einsum("lhd,hd->lh", k_full, q_full[b])
        out[b], lse[b] = _softmax_attend(s, v_full)
    return out, lse


def combine_ref(partial_out: np.ndarray, partial_lse: np.ndarray):
    """Merge split-KV partial results by their log-sum-exp.

    partial_out [S, ..., Dv] holds each split's normalised output o_s, and
    partial_lse [S, ...] its lse_s (-inf marks an empty split).
    lse = log sum_s exp(lse_s);  o = sum_s exp(lse_s - lse) o_s.

    The pages say only that flash-decoding splits the KV along the sequence,
    computes a local softmax per split and merges the normalisers at the end
    (arganzheng.life section 5.2); this is the merge that makes the split
    result equal the unsplit one.
    """
    po = np.asarray(partial_out, np.float64)
    pl = np.asarray(partial_lse, np.float64)
    m = pl.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(pl), np.exp(pl - m_safe[None]), 0.0)    # [S, ...]
    z = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, z, 1.0)), NEG_INF)
    coef = np.where(finite[None], w / np.where(finite, z, 1.0)[None], 0.0)
    # an empty split's o_s is never read: its weight is exactly zero
    po_safe = np.where(np.isfinite(pl)[..., None], po, 0.0)
    out = np.einsum("s...,s...d->...d", coef, po_safe)
    return out, lse


# ----------------------------------------------------------------------------
# paged KV caches
# ----------------------------------------------------------------------------

def paged_rows_ref(pool: np.ndarray, table_row, page_size: int, seq_len: int) -> np.ndarray:
    """The first ``seq_len`` cached rows of one sequence held in a paged pool.

    The cache of a sequence is cut into fixed-size blocks of ``page_size``
    tokens that live anywhere in a shared pool [num_pages, page_size, ...];
    the sequence's block table maps its logical block j to a physical page,
    and the kernel consults that table when it reads the cache
    (arganzheng.life, section 6.1 on paging: PagedAttention's blocks of 16
    tokens by default, the logical-to-physical map looked up on every KV
    read). Token t is therefore row t mod page_size of page table_row[t //
    page_size]. Only the blocks that hold rows are read.
    """
    n_blocks = -(-int(seq_len) // page_size)
    pages = np.asarray(table_row[:n_blocks], dtype=np.int64)
    rows = pool[pages].reshape((n_blocks * page_size,) + pool.shape[2:])
    return rows[:seq_len]


def gqa_decode_paged_ref(q, k_pool, v_pool, block_table, page_size: int, seq_lens, scale: float,
                         window: int = 0):
    """GQA decode over paged K and V pools [num_pages, page_size, Hkv, D]:
    each sequence's rows are gathered in logical order (paged_rows_ref), then
    attended exactly as by gqa_decode_ref. With a sliding window w only rows
    [max(0, L - w), L) are gathered, so table entries of earlier blocks are
    never looked at."""
    seq_lens = np.asarray(seq_lens, np.int64)
    B = q.shape[0]
    L = int(max(1, seq_lens.max(initial=0)))
    k = np.zeros((B, L) + k_pool.shape[2:])
    v = np.zeros((B, L) + v_pool.shape[2:])
    for b in range(B):
        Lb = int(seq_lens[b])
        if window > 0:
            for t in range(max(0, Lb - window), Lb):
                page = int(block_table[b][t // page_size])
                k[b, t] = k_pool[page, t % page_size]
                v[b, t] = v_pool[page, t % page_size]
        else:
            k[b, :Lb] = paged_rows_ref(k_pool, block_table[b], page_size, Lb)
            v[b, :Lb] = paged_rows_ref(v_pool, block_table[b], page_size, Lb)
    return gqa_decode_ref(q, k, v, seq_lens, scale, window)


def mla_absorbed_paged_ref(q_nope, q_rope, cache_pool, block_table, page_size: int, seq_lens,
                           w_uk, w_uv, scale: float, kv_lora_rank: int = 512):
    """Absorbed MLA decode over a paged latent pool [num_pages, page_size,
    d_c + d_rope]: rows gathered as by paged_rows_ref, then mla_absorbed_ref."""
    seq_lens = np.asarray(seq_lens, np.int64)
    B = q_nope.shape[0]
    L = int(max(1, seq_lens.max(initial=0)))
    cache = np.zeros((B, L) + cache_pool.shape[2:])
    for b in range(B):
        Lb = int(seq_lens[b])
        cache[b, :Lb] = paged_rows_ref(cache_pool, block_table[b], page_size, Lb)
    return mla_absorbed_ref(q_nope, q_rope, cache, seq_lens, w_uk, w_uv, scale, kv_lora_rank)
