"""Closed-form KV-cache sizes, decode FLOPs and intensity -- TEST INFRASTRUCTURE ONLY.

Re-derived from the formulas the pages state in prose; the worked numbers the
pages print are stored in tests/golden and checked against these functions.
"""
from __future__ import annotations

from dataclasses import dataclass

KIB, MIB, GIB = 1024, 1024 ** 2, 1024 ** 3


@dataclass(frozen=True)
class AttnModel:
    """Attention shape of one model (per layer), in the pages' notation."""
    name: str
    layers: int
    n_heads: int          # query heads n_h
    n_kv_heads: int       # KV heads n_kv (GQA); n_h for MHA; 1 for MQA
    head_dim: int         # d_head (d_h); for MLA the nope part
    attn_type: str        # "mha" | "gqa" | "mqa" | "mla"
    kv_lora_rank: int = 0     # d_c
    qk_rope_dim: int = 0      # d_h^R


# Model shapes quoted on the pages.
LLAMA3_8B = AttnModel("Llama-3-8B", 32, 32, 8, 128, "gqa")      # arganzheng.life section 1.1
LLAMA3_70B = AttnModel("Llama-3-70B", 80, 64, 8, 128, "gqa")    # arganzheng.life section 1.1
DEEPSEEK_V3 = AttnModel("DeepSeek-V3", 61, 128, 128, 128, "mla", 512, 64)  # arganzheng.life 4.2
LLAMA2_7B = AttnModel("LlaMA-2-7B", 32, 32, 32, 128, "mha")     # AIFAQ page; kakack.github.io 5


def kv_elems_per_token_per_layer(m: AttnModel) -> int:
    """Cached elements per token per layer.

    MHA 2*n_h*d_h, GQA 2*n_kv*d_h, MQA 2*d_h (AIFAQ page, per-scheme element
    counts; arganzheng.life section 2.3); MLA d_c + d_rope, the latent plus the
    decoupled RoPE key shared by every head (AIFAQ page, decoupled RoPE cache;
    arganzheng.life section 4.3).
    """
    if m.attn_type == "mha":
        return 2 * m.n_heads * m.head_dim
    if m.attn_type == "gqa":
        return 2 * m.n_kv_heads * m.head_dim
    if m.attn_type == "mqa":
        return 2 * m.head_dim
    if m.attn_type == "mla":
        return m.kv_lora_rank + m.qk_rope_dim
    raise ValueError(m.attn_type)


def as_type(m: AttnModel, attn_type: str) -> AttnModel:
    return AttnModel(m.name, m.layers, m.n_heads, m.n_kv_heads, m.head_dim, attn_type,
                     m.kv_lora_rank, m.qk_rope_dim)


def kv_bytes_per_token(m: AttnModel, elem_bytes: int = 2) -> int:
    """All layers: layers * elements per layer * bytes per element
    (arganzheng.life section 2.3)."""
    return m.layers * kv_elems_per_token_per_layer(m) * elem_bytes


def kv_bytes(m: AttnModel, ctx: int, elem_bytes: int = 2) -> int:
    return kv_bytes_per_token(m, elem_bytes) * ctx


def decode_flops_per_cached_token(m: AttnModel) -> int:
    """Attention FLOPs per cached token per layer at decode.

    Every query head does one dot product with the key and one weighted add of
    the value, 2 FLOPs per dimension each (arganzheng.life sections 3.3 and
    4.6). For absorbed MLA the key is the full d_c + d_rope row and the value
    its first d_c columns.
    """
    if m.attn_type == "mla":
        return m.n_heads * 2 * ((m.kv_lora_rank + m.qk_rope_dim) + m.kv_lora_rank)
    return m.n_heads * 2 * (m.head_dim + m.head_dim)


def decode_bytes_per_cached_token(m: AttnModel, elem_bytes: int = 2) -> int:
    return kv_elems_per_token_per_layer(m) * elem_bytes


def decode_intensity(m: AttnModel, elem_bytes: int = 2) -> float:
    """FLOP per byte of cache read (arganzheng.life sections 3.3 and 4.6)."""
    return decode_flops_per_cached_token(m) / decode_bytes_per_cached_token(m, elem_bytes)


def mla_mha_read_ratio(s: int, d_c: int = 512, d_h: int = 128, n_h: int = 128) -> float:
    """Absorbed-MLA vs MHA decode memory reads, q included, RoPE dims left out,
    as printed on the jianzhnie.github.io MLA page, section 4.2.3:
    M_MLA = 2 b d_c (n_h + s), M_MHA = 2 b d_h n_h (1 + s)."""
    return d_c * (n_h + s) / (d_h * n_h * (1 + s))


def mla_compute_bound_head_threshold(peak_flops: float, bandwidth: float) -> float:
    """Head count above which absorbed MLA decode is compute-bound:
    FLOPs ~ 4 n_h L d_c against bytes ~ 2 L d_c gives n_h > 2 Peak / (4 BW)
    (AIFAQ page, head-count threshold paragraph)."""
    return 2.0 * peak_flops / (4.0 * bandwidth)


def naive_upprojection_flops(L: int, d_c: int, d_model: int) -> int:
    """Decompressing L latents to K and V: 2 GEMMs of 2 L d_c d_model FLOPs each
    (AIFAQ page, up-projection cost paragraph)."""
    return 4 * L * d_c * d_model
