"""Closed-form cache sizes, decode work and intensity -- TEST INFRASTRUCTURE ONLY.

What one attention layer keeps per token is described as a list of cached
vectors, (how many, width): K and V of every KV head for the head-sharing
schemes, or one latent row and one decoupled RoPE key shared by all heads
for MLA. Every size and intensity below is a sum over that list. MHA, GQA
and MQA are not separate cases here: they differ only in the KV head count
(equal to the query heads, a divisor of them, or 1). The worked numbers the
pages print are stored in tests/golden and checked against these functions.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

# byte units used by the pages' worked numbers (binary prefixes)
UNIT = {"B": 1, "KiB": 1 << 10, "MiB": 1 << 20, "GiB": 1 << 30}


def in_unit(n_bytes: float, unit: str) -> float:
    return n_bytes / UNIT[unit]


@dataclass(frozen=True)
class Layer:
    """One attention layer in the pages' notation.

    q_heads n_h; kv_heads n_kv (n_h for MHA, a divisor for GQA, 1 for MQA;
    unused with a latent cache); head_dim d_h (for MLA the no-RoPE part of a
    query head); latent d_c and rope d_h^R, both 0 unless the layer caches a
    latent row (MLA)."""
    q_heads: int
    kv_heads: int
    head_dim: int
    latent: int = 0
    rope: int = 0


@dataclass(frozen=True)
class Model:
    name: str
    depth: int          # layers
    layer: Layer


# Shapes quoted on the pages.
LLAMA3_8B = Model("Llama-3-8B", 32, Layer(32, 8, 128))            # arganzheng.life section 1.1
LLAMA3_70B = Model("Llama-3-70B", 80, Layer(64, 8, 128))          # arganzheng.life section 1.1
DEEPSEEK_V3 = Model("DeepSeek-V3", 61, Layer(128, 128, 128, 512, 64))  # arganzheng.life section 4.2
LLAMA2_7B = Model("LlaMA-2-7B", 32, Layer(32, 32, 128))           # AIFAQ page; kakack.github.io section 5


def with_kv_heads(m: Model, kv_heads: int) -> Model:
    """The same model caching plain K and V for ``kv_heads`` KV heads (no
    latent): kv_heads = q_heads is its MHA form, 1 its MQA form."""
    return replace(m, layer=replace(m.layer, kv_heads=kv_heads, latent=0, rope=0))


def cached_vectors(layer: Layer):
    """(count, width) of every vector one layer caches per token.

    Head sharing caches a key and a value per KV head: 2 n_kv d_h elements,
    i.e. 2 n_h d_h for MHA and 2 d_h for MQA (AIFAQ page, per-scheme element
    counts; arganzheng.life section 2.3). MLA caches the latent c_kv (d_c)
    and the decoupled RoPE key (d_h^R), each once for all heads (AIFAQ page,
    decoupled-RoPE cache; arganzheng.life section 4.3)."""
    if layer.latent:
        return ((1, layer.latent), (1, layer.rope))
    keys = (layer.kv_heads, layer.head_dim)
    values = (layer.kv_heads, layer.head_dim)
    return (keys, values)


def elements_per_token(layer: Layer) -> int:
    """Cached elements per token in one layer."""
    return sum(count * width for count, width in cached_vectors(layer))


def cache_bytes(m: Model, tokens: int = 1, elem_bytes: int = 2) -> int:
    """Cache of ``tokens`` tokens over all layers: depth x elements per token
    per layer x element bytes x tokens (arganzheng.life section 2.3)."""
    return m.depth * elements_per_token(m.layer) * elem_bytes * tokens


def row_bytes(layer: Layer, elem_bytes: int = 2) -> int:
    """Bytes of one cached token of one layer: what decode reads per cached row."""
    return elements_per_token(layer) * elem_bytes


def row_flops(layer: Layer) -> int:
    """Attention FLOPs per cached token per layer at decode.

    Each query head takes one dot product with the row's key and adds the
    row's value with its weight, 2 FLOPs per element each (arganzheng.life
    sections 3.3 and 4.6). With a latent cache the key is the whole
    d_c + d_h^R row and the value its first d_c elements; otherwise both are
    d_h wide."""
    L = layer
    key_width = L.latent + L.rope if L.latent else L.head_dim
    value_width = L.latent if L.latent else L.head_dim
    return L.q_heads * 2 * (key_width + value_width)


def intensity(layer: Layer, elem_bytes: int = 2) -> float:
    """FLOP per byte of cache read at decode (arganzheng.life sections 3.3 and 4.6)."""
    return row_flops(layer) / row_bytes(layer, elem_bytes)


def mla_mha_read_ratio(s: int, d_c: int = 512, d_h: int = 128, n_h: int = 128) -> float:
    """Absorbed-MLA over MHA decode memory reads, the query included and the
    RoPE dims left out, as the jianzhnie.github.io MLA page (section 4.2.3)
    counts them: MLA reads 2 b d_c (n_h + s), MHA 2 b d_h n_h (1 + s)."""
    mla = d_c * (n_h + s)
    mha = d_h * n_h * (1 + s)
    return mla / mha


def mla_compute_bound_head_threshold(peak_flops: float, bandwidth: float) -> float:
    """Head count above which absorbed MLA decode is compute-bound: about
    4 n_h L d_c FLOPs against 2 L d_c bytes, so n_h > 2 Peak / (4 BW)
    (AIFAQ page, head-count threshold paragraph)."""
    return 2.0 * peak_flops / (4.0 * bandwidth)


def naive_upprojection_flops(L: int, d_c: int, d_model: int) -> int:
    """Decompressing L latents into K and V: two products of 2 L d_c d_model
    FLOPs each (AIFAQ page, up-projection cost paragraph)."""
    per_product = 2 * L * d_c * d_model
    return 2 * per_product
