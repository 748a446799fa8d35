"""Decode attention over a KV cache on AMD MI355X: Python binding.

A thin ctypes layer over libdecode_attn.so (see include/decode_attn.h). It
only marshals arguments: it reads tensor pointers, shapes and strides,
allocates outputs and workspace through PyTorch's caching allocator and passes
the current HIP stream. Every step of the computation runs in the library's
HIP kernels; there is no fallback. If the library is missing, every call
raises.

    out, lse = gqa_decode(q, k_cache, v_cache, seq_lens)
    out, lse = mla_decode_absorbed(q_nope, q_rope, kv_cache, w_uk, w_uv, seq_lens)
    out, lse = splitkv_combine(partial_out, partial_lse)
    out, lse = gqa_decode_paged(q, k_pool, v_pool, block_table, page_size, seq_lens)
    out, lse = gqa_decode_fp8(q, k_codes, v_codes, k_scale, v_scale, seq_lens)
    out, lse = mla_decode_absorbed_paged(q_nope, q_rope, cache_pool, block_table, page_size,
                                         seq_lens, w_uk, w_uv)
    q_rot = gqa_append_rope(q, k_new, v_new, positions, k_cache, v_cache)
    q_rope_rot = mla_append_rope(q_rope, kv_new, positions, kv_cache)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libdecode_attn.so")

DA_OK = 0
DA_DTYPE_F32 = 0
DA_DTYPE_BF16 = 1
DA_DTYPE_FP8_E4M3 = 2


class GqaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_stride_b", ctypes.c_int64),
        ("q_stride_h", ctypes.c_int64),
        ("kv_stride_b", ctypes.c_int64),
        ("kv_stride_t", ctypes.c_int64),
        ("kv_stride_h", ctypes.c_int64),
        ("num_splits", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32),
    ]


class MlaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("qk_rope_dim", ctypes.c_int32),
        ("qk_nope_dim", ctypes.c_int32),
        ("v_head_dim", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("cache_stride_b", ctypes.c_int64),
        ("cache_stride_t", ctypes.c_int64),
        ("num_splits", ctypes.c_int32),
    ]


class PagedKv(ctypes.Structure):
    _fields_ = [
        ("block_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("page_stride", ctypes.c_int64),
    ]


class KvScales(ctypes.Structure):
    _fields_ = [
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("stride_b", ctypes.c_int64),
        ("stride_t", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
    ]


class MlaScales(ctypes.Structure):
    _fields_ = [
        ("nope_scale", ctypes.c_void_p),
        ("rope_scale", ctypes.c_void_p),
        ("stride_b", ctypes.c_int64),
        ("stride_t", ctypes.c_int64),
    ]


ROPE_STYLES = {"half": 0, "interleaved": 1}


class Append(ctypes.Structure):
    _fields_ = [
        ("rotary_dim", ctypes.c_int32),
        ("rope_style", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("inv_freq", ctypes.c_void_p),
        ("new_stride_b", ctypes.c_int64),
        ("new_stride_h", ctypes.c_int64),
    ]


_vp = ctypes.c_void_p
_GQA_P = ctypes.POINTER(GqaParams)
_MLA_P = ctypes.POINTER(MlaParams)
_PAGED_P = ctypes.POINTER(PagedKv)
_SIGNATURES = {
    "da_gqa_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(GqaParams)]),
    "da_gqa_decode_num_splits": (ctypes.c_int32, [ctypes.POINTER(GqaParams)]),
    "da_gqa_decode_split_pass": (ctypes.c_int, [ctypes.POINTER(GqaParams), _vp, _vp, _vp, _vp, _vp,
                                                _vp, _vp]),
    "da_gqa_decode": (ctypes.c_int, [ctypes.POINTER(GqaParams), _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, ctypes.c_size_t, _vp]),
    "da_mla_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MlaParams)]),
    "da_mla_decode_num_splits": (ctypes.c_int32, [ctypes.POINTER(MlaParams)]),
    "da_mla_partials_size": (ctypes.c_int, [ctypes.POINTER(MlaParams), ctypes.POINTER(ctypes.c_size_t),
                                            ctypes.POINTER(ctypes.c_size_t)]),
    "da_mla_decode_absorbed": (ctypes.c_int, [ctypes.POINTER(MlaParams), _vp, _vp, _vp, _vp, _vp,
                                              _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "da_mla_absorb_query": (ctypes.c_int, [ctypes.POINTER(MlaParams), _vp, _vp, _vp, _vp, _vp]),
    "da_mla_attend_split_pass": (ctypes.c_int, [ctypes.POINTER(MlaParams), _vp, _vp, _vp, _vp,
                                                _vp, _vp]),
    "da_mla_decode_absorbed_noalloc": (ctypes.c_int, [ctypes.POINTER(MlaParams), _vp, _vp, _vp, _vp, _vp,
                                                      _vp, _vp, _vp, _vp]),
    "da_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "da_mla_decode_fp8_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MlaParams)]),
    "da_mla_decode_absorbed_fp8": (ctypes.c_int, [_MLA_P, ctypes.POINTER(MlaScales), _vp, _vp, _vp, _vp,
                                                  _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "da_mla_decode_absorbed_fp8_paged": (ctypes.c_int, [_MLA_P, _PAGED_P, ctypes.POINTER(MlaScales), _vp, _vp,
                                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                                        _vp]),
    "da_mla_merge_project": (ctypes.c_int, [ctypes.POINTER(MlaParams), _vp, _vp, _vp, _vp, _vp,
                                            _vp, _vp]),
    "da_gqa_decode_paged": (ctypes.c_int, [_GQA_P, _PAGED_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           ctypes.c_size_t, _vp]),
    "da_mla_decode_absorbed_paged": (ctypes.c_int, [_MLA_P, _PAGED_P, _vp, _vp, _vp, _vp, _vp, _vp,
                                                    _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "da_mla_attend_split_pass_paged": (ctypes.c_int, [_MLA_P, _PAGED_P, _vp, _vp, _vp, _vp, _vp,
                                                      _vp]),
    "da_gqa_decode_fp8": (ctypes.c_int, [_GQA_P, ctypes.POINTER(KvScales), _vp, _vp, _vp, _vp, _vp,
                                         _vp, _vp, ctypes.c_size_t, _vp]),
    "da_gqa_append_rope": (ctypes.c_int, [_GQA_P, ctypes.POINTER(Append), _PAGED_P, _vp, _vp, _vp,
                                          _vp, _vp, _vp, _vp, _vp]),
    "da_gqa_append_rope_fp8": (ctypes.c_int, [_GQA_P, ctypes.POINTER(Append), _PAGED_P,
                                              ctypes.POINTER(KvScales), _vp, _vp, _vp, _vp, _vp, _vp,
                                              _vp, _vp]),
    "da_mla_append_rope": (ctypes.c_int, [_MLA_P, ctypes.POINTER(Append), _PAGED_P, _vp, _vp, _vp,
                                          _vp, _vp, _vp]),
    "da_gqa_decode_fp8_paged": (ctypes.c_int, [_GQA_P, _PAGED_P, ctypes.POINTER(KvScales), _vp, _vp, _vp,
                                               _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "da_splitkv_combine": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]),
    "da_probe_stream_read": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                            _vp, _vp]),
    "da_probe_stream_copy": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_int32, _vp]),
    "da_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "da_version": (ctypes.c_int32, []),
    "da_gqa_params_size": (ctypes.c_size_t, []),
    "da_mla_params_size": (ctypes.c_size_t, []),
    "da_paged_kv_size": (ctypes.c_size_t, []),
    "da_kv_scales_size": (ctypes.c_size_t, []),
    "da_mla_scales_size": (ctypes.c_size_t, []),
    "da_append_size": (ctypes.c_size_t, []),
}

_lib: Optional[ctypes.CDLL] = None


class LibraryMissing(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use). Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is not built; run `python -m decode_attention_kv_bf16_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    if L.da_gqa_params_size() != ctypes.sizeof(GqaParams) or \
            L.da_mla_params_size() != ctypes.sizeof(MlaParams) or \
            L.da_paged_kv_size() != ctypes.sizeof(PagedKv) or \
            L.da_kv_scales_size() != ctypes.sizeof(KvScales) or \
            L.da_mla_scales_size() != ctypes.sizeof(MlaScales) or \
            L.da_append_size() != ctypes.sizeof(Append):
        raise RuntimeError("libdecode_attn.so parameter structs do not match this binding")
    _lib = L
    return L


_recorder: Optional[list] = None


def _call(name: str, *args) -> int:
    """Call a library entry point; inside recorded_calls() also record it."""
    fn = getattr(lib(), name)
    if _recorder is not None:
        _recorder.append((fn, args))
    return fn(*args)


class recorded_calls:
    """Records every library call made by the wrappers inside the block as
    (C function, ctypes arguments). Calling fn(*args) later repeats exactly
    that call (same buffers, parameters and stream) without the wrapper's
    Python work, which matters for kernels that take a few microseconds. The
    tensors the call used must stay alive for as long as it is replayed."""

    def __enter__(self):
        global _recorder
        self.calls = []
        _recorder = self.calls
        return self.calls

    def __exit__(self, *exc):
        global _recorder
        _recorder = None
        return False


def loaded_library_path() -> Optional[str]:
    return LIB_PATH if _lib is not None else None


class DecodeAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib().da_status_string(status).decode()
        super().__init__(f"{what}: {msg} (status {status})")
        self.status = status


def _check(status: int, what: str):
    if status != DA_OK:
        raise DecodeAttnError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _require_cuda(name: str, t: torch.Tensor):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------
# GQA / MQA / MHA
# ----------------------------------------------------------------------------

def gqa_params(q: torch.Tensor, k_cache: torch.Tensor, softmax_scale: Optional[float] = None,
               num_splits: int = 0, window: int = 0) -> GqaParams:
    B, Hq, D = q.shape
    Bk, L_max, Hkv, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError(f"q {tuple(q.shape)} and cache {tuple(k_cache.shape)} disagree")
    if q.dtype == torch.bfloat16:
        dt = DA_DTYPE_BF16
    elif q.dtype == torch.float32:
        dt = DA_DTYPE_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q.stride(2) != 1 or k_cache.stride(3) != 1:
        raise ValueError("the head_dim axis must be contiguous")
    p = GqaParams()
    p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.max_seq_len = B, Hq, Hkv, D, L_max
    p.dtype = dt
    p.softmax_scale = (1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale)
    p.q_stride_b, p.q_stride_h = q.stride(0), q.stride(1)
    p.kv_stride_b, p.kv_stride_t, p.kv_stride_h = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    p.num_splits = int(num_splits)
    p.sliding_window = int(window)
    return p


def gqa_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               seq_lens: Optional[torch.Tensor] = None, softmax_scale: Optional[float] = None,
               num_splits: int = 0, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, window: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """GQA/MQA/MHA decode of one new token per sequence.

    q [B, Hq, D]; k_cache, v_cache [B, L_max, Hkv, D] (same dtype, bf16 or fp32,
    same strides); seq_lens [B] int32 on the GPU (None: all L_max).
    Returns out [B, Hq, D] float32 and lse [B, Hq] float32 (natural log).
    window w > 0: sliding-window attention over the last w rows of each sequence.
    """
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _require_cuda(name, t)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, k_cache and v_cache must share a dtype")
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("v_cache must have the shape and strides of k_cache")
    if seq_lens is not None:
        _require_cuda("seq_lens", seq_lens)
        if seq_lens.dtype != torch.int32 or seq_lens.shape != (q.shape[0],) or not seq_lens.is_contiguous():
            raise ValueError("seq_lens must be a contiguous int32 tensor of shape [B]")
    p = gqa_params(q, k_cache, softmax_scale, num_splits, window)
    L = lib()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws_bytes = L.da_gqa_decode_workspace_size(ctypes.byref(p))
    ws = _workspace(ws_bytes, q.device)
    st = L.da_gqa_decode(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                         _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream_handle())
    _check(st, "da_gqa_decode")
    return out, lse


def gqa_decode_split_pass(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          seq_lens: Optional[torch.Tensor] = None,
                          softmax_scale: Optional[float] = None, num_splits: int = 0,
                          part_out: Optional[torch.Tensor] = None,
                          part_lse: Optional[torch.Tensor] = None, window: int = 0):
    """The split pass alone: returns per-split (part_out [S,B,Hq,D], part_lse [S,B,Hq]).
    splitkv_combine() of these equals gqa_decode()."""
    p = gqa_params(q, k_cache, softmax_scale, num_splits, window)
    L = lib()
    S = int(L.da_gqa_decode_num_splits(ctypes.byref(p)))
    B, Hq, D = q.shape
    if part_out is None:
        part_out = torch.empty((S, B, Hq, D), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((S, B, Hq), dtype=torch.float32, device=q.device)
    st = L.da_gqa_decode_split_pass(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(seq_lens), _ptr(part_out), _ptr(part_lse),
                                    _stream_handle())
    _check(st, "da_gqa_decode_split_pass")
    return part_out, part_lse


def gqa_num_splits(q: torch.Tensor, k_cache: torch.Tensor, num_splits: int = 0, window: int = 0) -> int:
    p = gqa_params(q, k_cache, None, num_splits, window)
    return int(lib().da_gqa_decode_num_splits(ctypes.byref(p)))


# ----------------------------------------------------------------------------
# FP8 (E4M3) caches
# ----------------------------------------------------------------------------

def gqa_decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   k_scale: torch.Tensor, v_scale: torch.Tensor,
                   seq_lens: Optional[torch.Tensor] = None, softmax_scale: Optional[float] = None,
                   num_splits: int = 0, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, window: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """gqa_decode over an E4M3 cache: q [B, Hq, D] bf16; k_cache, v_cache
    [B, L_max, Hkv, D] uint8 codes (or torch.float8_e4m3fn); k_scale, v_scale
    float32 of shape [B, L_max, Hkv] (broadcast views with zero strides are
    fine: per token, per head). Element (b, t, h, :) of K stands for its code's
    value times k_scale[b, t, h]."""
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("k_scale", k_scale),
                    ("v_scale", v_scale)):
        _require_cuda(name, t)
    if q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16")
    if k_cache.dtype == torch.float8_e4m3fn:
        k_cache, v_cache = k_cache.view(torch.uint8), v_cache.view(torch.uint8)
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("k_cache and v_cache must hold E4M3 codes (uint8 or float8_e4m3fn)")
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("v_cache must have the shape and strides of k_cache")
    B, Hq, D = q.shape
    Bk, L_max, Hkv, Dk = k_cache.shape
    if Bk != B or Dk != D or q.stride(2) != 1 or k_cache.stride(3) != 1:
        raise ValueError("q and the cache disagree, or the head_dim axis is not contiguous")
    for name, s in (("k_scale", k_scale), ("v_scale", v_scale)):
        if s.dtype != torch.float32 or s.shape != (B, L_max, Hkv):
            raise ValueError(f"{name} must be float32 of shape [B, L_max, Hkv]")
    if k_scale.stride() != v_scale.stride():
        raise ValueError("k_scale and v_scale must share strides")
    if seq_lens is not None:
        _check_seq_lens(seq_lens, B)
    p = GqaParams()
    p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.max_seq_len = B, Hq, Hkv, D, L_max
    p.dtype = DA_DTYPE_FP8_E4M3
    p.softmax_scale = (1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale)
    p.q_stride_b, p.q_stride_h = q.stride(0), q.stride(1)
    p.kv_stride_b, p.kv_stride_t, p.kv_stride_h = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    p.num_splits = int(num_splits)
    p.sliding_window = int(window)
    sc = KvScales()
    sc.k_scale, sc.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
    sc.stride_b, sc.stride_t, sc.stride_h = k_scale.stride()
    L = lib()
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws_bytes = L.da_gqa_decode_workspace_size(ctypes.byref(p))
    ws = _workspace(ws_bytes, q.device)
    st = L.da_gqa_decode_fp8(ctypes.byref(p), ctypes.byref(sc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                             _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream_handle())
    _check(st, "da_gqa_decode_fp8")
    return out, lse


# ----------------------------------------------------------------------------
# paged pools
# ----------------------------------------------------------------------------

def gqa_decode_fp8_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                         k_scale: torch.Tensor, v_scale: torch.Tensor, block_table: torch.Tensor,
                         page_size: int, seq_lens: torch.Tensor, max_seq_len: Optional[int] = None,
                         softmax_scale: Optional[float] = None, num_splits: int = 0,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         window: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """gqa_decode_fp8 over paged E4M3 pools: k_pool, v_pool [num_pages,
    page_size, Hkv, D] uint8 codes (page_size >= 32); k_scale, v_scale
    float32 [num_pages, page_size, Hkv] (or a per-head [Hkv] vector expanded
    with zero strides); block_table [B, max_blocks] int32; seq_lens [B] int32."""
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("k_scale", k_scale),
                    ("v_scale", v_scale)):
        _require_cuda(name, t)
    if q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16")
    if k_pool.dtype == torch.float8_e4m3fn:
        k_pool, v_pool = k_pool.view(torch.uint8), v_pool.view(torch.uint8)
    if k_pool.dtype != torch.uint8 or v_pool.dtype != torch.uint8:
        raise ValueError("k_pool and v_pool must hold E4M3 codes (uint8 or float8_e4m3fn)")
    if v_pool.shape != k_pool.shape or v_pool.stride() != k_pool.stride() or k_pool.stride(3) != 1:
        raise ValueError("v_pool must have the shape and strides of k_pool, with a contiguous D axis")
    n_pages, ps, Hkv, D = k_pool.shape
    for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
        if sc.dtype != torch.float32 or sc.shape != (n_pages, ps, Hkv):
            raise ValueError(f"{name} must be float32 of shape [num_pages, page_size, Hkv]")
    if k_scale.stride() != v_scale.stride():
        raise ValueError("k_scale and v_scale must share strides")
    B, Hq, Dq = q.shape
    if Dq != D or q.stride(2) != 1:
        raise ValueError("q and the pools disagree, or the head_dim axis is not contiguous")
    _check_seq_lens(seq_lens, B)
    pg = paged_kv(block_table, page_size, k_pool)
    if block_table.shape[0] != B:
        raise ValueError("block_table must have one row per sequence")
    p = GqaParams()
    p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim = B, Hq, Hkv, D
    p.max_seq_len = block_table.shape[1] * page_size if max_seq_len is None else int(max_seq_len)
    p.dtype = DA_DTYPE_FP8_E4M3
    p.softmax_scale = (1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale)
    p.q_stride_b, p.q_stride_h = q.stride(0), q.stride(1)
    p.kv_stride_b, p.kv_stride_t, p.kv_stride_h = 0, k_pool.stride(1), k_pool.stride(2)
    p.num_splits = int(num_splits)
    p.sliding_window = int(window)
    sc = KvScales()
    sc.k_scale, sc.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
    sc.stride_b, sc.stride_t, sc.stride_h = k_scale.stride()
    L = lib()
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws_bytes = L.da_gqa_decode_workspace_size(ctypes.byref(p))
    ws = _workspace(ws_bytes, q.device)
    st = L.da_gqa_decode_fp8_paged(ctypes.byref(p), ctypes.byref(pg), ctypes.byref(sc), _ptr(q),
                                   _ptr(k_pool), _ptr(v_pool), _ptr(seq_lens), _ptr(out), _ptr(lse),
                                   _ptr(ws), ws_bytes, _stream_handle())
    _check(st, "da_gqa_decode_fp8_paged")
    return out, lse


def paged_kv(block_table: torch.Tensor, page_size: int, pool: torch.Tensor) -> PagedKv:
    """The paging descriptor for a pool [num_pages, page_size, ...] and a
    block table [B, max_blocks_per_seq] int32 on the GPU."""
    _require_cuda("block_table", block_table)
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 tensor [B, max_blocks_per_seq]")
    if pool.shape[1] != page_size:
        raise ValueError(f"pool pages hold {pool.shape[1]} rows, page_size is {page_size}")
    pg = PagedKv()
    pg.block_table = block_table.data_ptr()
    pg.page_size = int(page_size)
    pg.max_blocks_per_seq = block_table.shape[1]
    pg.page_stride = pool.stride(0)
    return pg


def _check_seq_lens(seq_lens: torch.Tensor, B: int):
    _require_cuda("seq_lens", seq_lens)
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of shape [B]")


def gqa_decode_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                     block_table: torch.Tensor, page_size: int, seq_lens: torch.Tensor,
                     max_seq_len: Optional[int] = None, softmax_scale: Optional[float] = None,
                     num_splits: int = 0, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, window: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """gqa_decode over paged pools: k_pool, v_pool [num_pages, page_size, Hkv, D];
    block_table [B, max_blocks_per_seq] int32 (token t of sequence b is row
    t % page_size of page block_table[b, t // page_size]); seq_lens [B] int32.
    max_seq_len (default: the table's capacity) bounds every seq_lens[b]."""
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _require_cuda(name, t)
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise ValueError("q, k_pool and v_pool must share a dtype")
    if v_pool.shape != k_pool.shape or v_pool.stride() != k_pool.stride():
        raise ValueError("v_pool must have the shape and strides of k_pool")
    B = q.shape[0]
    _check_seq_lens(seq_lens, B)
    pg = paged_kv(block_table, page_size, k_pool)
    if block_table.shape[0] != B:
        raise ValueError("block_table must have one row per sequence")
    if max_seq_len is None:
        max_seq_len = block_table.shape[1] * page_size
    if k_pool.shape[3] != q.shape[2] or k_pool.stride(3) != 1:
        raise ValueError("k_pool must be [num_pages, page_size, Hkv, D] with a contiguous D axis")
    # the params describe a [B, max_seq_len, Hkv, D] cache with the pool's
    # token and head strides (the batch stride is unused for paged pools)
    p = gqa_params(q, k_pool[:1].expand(B, -1, -1, -1), softmax_scale, num_splits, window)
    p.max_seq_len = int(max_seq_len)
    p.kv_stride_b = 0
    L = lib()
    Hq, D = q.shape[1], q.shape[2]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws_bytes = L.da_gqa_decode_workspace_size(ctypes.byref(p))
    ws = _workspace(ws_bytes, q.device)
    st = L.da_gqa_decode_paged(ctypes.byref(p), ctypes.byref(pg), _ptr(q), _ptr(k_pool),
                               _ptr(v_pool), _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(ws),
                               ws_bytes, _stream_handle())
    _check(st, "da_gqa_decode_paged")
    return out, lse


# ----------------------------------------------------------------------------
# absorbed MLA
# ----------------------------------------------------------------------------

def mla_params(q_nope: torch.Tensor, kv_cache: torch.Tensor, w_uv: torch.Tensor,
               q_rope: torch.Tensor, softmax_scale: Optional[float] = None,
               num_splits: int = 0) -> MlaParams:
    B, H, d_nope = q_nope.shape
    Bc, L_max, row = kv_cache.shape
    d_rope = q_rope.shape[2]
    d_c = row - d_rope
    if Bc != B:
        raise ValueError("q_nope and kv_cache disagree on the batch size")
    if kv_cache.stride(2) != 1:
        raise ValueError("kv_cache rows must be contiguous")
    p = MlaParams()
    p.batch, p.num_heads, p.kv_lora_rank, p.qk_rope_dim = B, H, d_c, d_rope
    p.qk_nope_dim, p.v_head_dim, p.max_seq_len = d_nope, w_uv.shape[2], L_max
    p.softmax_scale = (1.0 / math.sqrt(d_nope + d_rope)) if softmax_scale is None else float(softmax_scale)
    p.cache_stride_b, p.cache_stride_t = kv_cache.stride(0), kv_cache.stride(1)
    p.num_splits = int(num_splits)
    return p


def mla_decode_absorbed(q_nope: torch.Tensor, q_rope: torch.Tensor, kv_cache: torch.Tensor,
                        w_uk: torch.Tensor, w_uv: torch.Tensor,
                        seq_lens: Optional[torch.Tensor] = None,
                        softmax_scale: Optional[float] = None, num_splits: int = 0,
                        out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """DeepSeek-style absorbed MLA decode of one new token per sequence.

    q_nope [B,H,128], q_rope [B,H,64], kv_cache [B,L_max,576] (row = [c_kv | k_rope]),
    w_uk, w_uv [H,512,128] -- all bf16; seq_lens [B] int32 on the GPU or None.
    Returns out [B,H,128] float32 and lse [B,H] float32.
    """
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("kv_cache", kv_cache),
                    ("w_uk", w_uk), ("w_uv", w_uv)):
        _require_cuda(name, t)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("w_uk", w_uk), ("w_uv", w_uv)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, _ = q_nope.shape
    if q_rope.shape[:2] != (B, H) or w_uk.shape[0] != H or w_uv.shape[0] != H:
        raise ValueError("head counts disagree")
    if w_uk.shape[1] != kv_cache.shape[2] - q_rope.shape[2] or w_uk.shape[2] != q_nope.shape[2]:
        raise ValueError("w_uk must be [H, d_c, d_nope]")
    if w_uv.shape[1] != w_uk.shape[1]:
        raise ValueError("w_uv must be [H, d_c, d_v]")
    if seq_lens is not None:
        _require_cuda("seq_lens", seq_lens)
        if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,) or not seq_lens.is_contiguous():
            raise ValueError("seq_lens must be a contiguous int32 tensor of shape [B]")
    p = mla_params(q_nope, kv_cache, w_uv, q_rope, softmax_scale, num_splits)
    L = lib()
    if out is None:
        out = torch.empty((B, H, w_uv.shape[2]), dtype=torch.float32, device=q_nope.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device)
    ws_bytes = L.da_mla_decode_workspace_size(ctypes.byref(p))
    ws = _workspace(ws_bytes, q_nope.device)
    st = L.da_mla_decode_absorbed(ctypes.byref(p), _ptr(q_nope), _ptr(q_rope), _ptr(kv_cache),
                                  _ptr(seq_lens), _ptr(w_uk), _ptr(w_uv), _ptr(out), _ptr(lse),
                                  _ptr(ws), ws_bytes, _stream_handle())
    _check(st, "da_mla_decode_absorbed")
    return out, lse


def mla_decode_absorbed_fp8(q_nope: torch.Tensor, q_rope: torch.Tensor, kv_codes: torch.Tensor,
                            scale_nope: torch.Tensor, scale_rope: torch.Tensor,
                            w_uk: torch.Tensor, w_uv: torch.Tensor,
                            seq_lens: Optional[torch.Tensor] = None,
                            softmax_scale: Optional[float] = None, num_splits: int = 0,
                            out: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_decode_absorbed over an E4M3 latent cache: kv_codes [B, L_max, 576]
    uint8 codes (or torch.float8_e4m3fn); scale_nope, scale_rope float32
    [B, L_max] (zero-stride views are fine): row (b, t) stands for
    [code[:512] * scale_nope[b, t] ; code[512:] * scale_rope[b, t]]. The other
    arguments as for mla_decode_absorbed."""
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("kv_codes", kv_codes),
                    ("scale_nope", scale_nope), ("scale_rope", scale_rope), ("w_uk", w_uk), ("w_uv", w_uv)):
        _require_cuda(name, t)
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("w_uk", w_uk), ("w_uv", w_uv)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if kv_codes.dtype == torch.float8_e4m3fn:
        kv_codes = kv_codes.view(torch.uint8)
    if kv_codes.dtype != torch.uint8:
        raise ValueError("kv_codes must hold E4M3 codes (uint8 or float8_e4m3fn)")
    B, H, _ = q_nope.shape
    if q_rope.shape[:2] != (B, H) or w_uk.shape[0] != H or w_uv.shape[0] != H:
        raise ValueError("head counts disagree")
    L_max = kv_codes.shape[1]
    for name, sc in (("scale_nope", scale_nope), ("scale_rope", scale_rope)):
        if sc.dtype != torch.float32 or sc.shape != (B, L_max):
            raise ValueError(f"{name} must be float32 of shape [B, L_max]")
    if scale_nope.stride() != scale_rope.stride():
        raise ValueError("scale_nope and scale_rope must share strides")
    if seq_lens is not None:
        _check_seq_lens(seq_lens, B)
    p = mla_params(q_nope, kv_codes, w_uv, q_rope, softmax_scale, num_splits)
    sc = MlaScales()
    sc.nope_scale, sc.rope_scale = scale_nope.data_ptr(), scale_rope.data_ptr()
    sc.stride_b, sc.stride_t = scale_nope.stride()
    L = lib()
    if out is None:
        out = torch.empty((B, H, w_uv.shape[2]), dtype=torch.float32, device=q_nope.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device)
    ws_bytes = L.da_mla_decode_fp8_workspace_size(ctypes.byref(p))
    ws = _workspace(ws_bytes, q_nope.device)
    st = L.da_mla_decode_absorbed_fp8(ctypes.byref(p), ctypes.byref(sc), _ptr(q_nope), _ptr(q_rope),
                                      _ptr(kv_codes), _ptr(seq_lens), _ptr(w_uk), _ptr(w_uv), _ptr(out),
                                      _ptr(lse), _ptr(ws), ws_bytes, _stream_handle())
    _check(st, "da_mla_decode_absorbed_fp8")
    return out, lse


def mla_decode_absorbed_fp8_paged(q_nope: torch.Tensor, q_rope: torch.Tensor, code_pool: torch.Tensor,
                                  scale_nope: torch.Tensor, scale_rope: torch.Tensor,
                                  block_table: torch.Tensor, page_size: int, seq_lens: torch.Tensor,
                                  w_uk: torch.Tensor, w_uv: torch.Tensor,
                                  max_seq_len: Optional[int] = None,
                                  softmax_scale: Optional[float] = None, num_splits: int = 0,
                                  out: Optional[torch.Tensor] = None,
                                  lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_decode_absorbed_fp8 over a paged E4M3 latent pool: code_pool
    [num_pages, page_size, 576] uint8 codes (or float8_e4m3fn); scale_nope,
    scale_rope float32 [num_pages, page_size] (paged like the codes; zero
    strides are fine); block_table [B, max_blocks] int32; seq_lens [B] int32."""
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("code_pool", code_pool),
                    ("scale_nope", scale_nope), ("scale_rope", scale_rope), ("w_uk", w_uk), ("w_uv", w_uv)):
        _require_cuda(name, t)
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("w_uk", w_uk), ("w_uv", w_uv)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if code_pool.dtype == torch.float8_e4m3fn:
        code_pool = code_pool.view(torch.uint8)
    if code_pool.dtype != torch.uint8:
        raise ValueError("code_pool must hold E4M3 codes (uint8 or float8_e4m3fn)")
    B, H, _ = q_nope.shape
    if q_rope.shape[:2] != (B, H) or w_uk.shape[0] != H or w_uv.shape[0] != H:
        raise ValueError("head counts disagree")
    for name, sc in (("scale_nope", scale_nope), ("scale_rope", scale_rope)):
        if sc.dtype != torch.float32 or sc.shape != tuple(code_pool.shape[:2]):
            raise ValueError(f"{name} must be float32 of shape [num_pages, page_size]")
    if scale_nope.stride() != scale_rope.stride():
        raise ValueError("scale_nope and scale_rope must share strides")
    _check_seq_lens(seq_lens, B)
    if block_table.shape[0] != B:
        raise ValueError("block_table must have one row per sequence")
    pg = paged_kv(block_table, page_size, code_pool)
    if max_seq_len is None:
        max_seq_len = block_table.shape[1] * page_size
    p = _mla_paged_params(q_nope, q_rope, code_pool, w_uv, max_seq_len, softmax_scale, num_splits)
    sc = MlaScales()
    sc.nope_scale, sc.rope_scale = scale_nope.data_ptr(), scale_rope.data_ptr()
    sc.stride_b, sc.stride_t = scale_nope.stride()
    L = lib()
    if out is None:
        out = torch.empty((B, H, w_uv.shape[2]), dtype=torch.float32, device=q_nope.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device)
    ws_bytes = L.da_mla_decode_fp8_workspace_size(ctypes.byref(p))
    ws = _workspace(ws_bytes, q_nope.device)
    st = L.da_mla_decode_absorbed_fp8_paged(ctypes.byref(p), ctypes.byref(pg), ctypes.byref(sc), _ptr(q_nope),
                                            _ptr(q_rope), _ptr(code_pool), _ptr(seq_lens), _ptr(w_uk),
                                            _ptr(w_uv), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                            _stream_handle())
    _check(st, "da_mla_decode_absorbed_fp8_paged")
    return out, lse


def mla_decode_absorbed_noalloc(q_nope: torch.Tensor, q_rope: torch.Tensor, kv_cache: torch.Tensor,
                                w_uk: torch.Tensor, w_uv: torch.Tensor,
                                seq_lens: Optional[torch.Tensor] = None,
                                softmax_scale: Optional[float] = None, num_splits: int = 0,
                                out: Optional[torch.Tensor] = None,
                                lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_decode_absorbed through da_mla_decode_absorbed_noalloc: no
    workspace is allocated (the library's built-in scratch serves). With out
    and lse given, the call allocates nothing at all."""
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("kv_cache", kv_cache),
                    ("w_uk", w_uk), ("w_uv", w_uv)):
        _require_cuda(name, t)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("w_uk", w_uk), ("w_uv", w_uv)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, _ = q_nope.shape
    if q_rope.shape[:2] != (B, H) or w_uk.shape[0] != H or w_uv.shape[0] != H:
        raise ValueError("head counts disagree")
    if seq_lens is not None:
        _check_seq_lens(seq_lens, B)
    p = mla_params(q_nope, kv_cache, w_uv, q_rope, softmax_scale, num_splits)
    if out is None:
        out = torch.empty((B, H, w_uv.shape[2]), dtype=torch.float32, device=q_nope.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device)
    st = lib().da_mla_decode_absorbed_noalloc(ctypes.byref(p), _ptr(q_nope), _ptr(q_rope), _ptr(kv_cache),
                                              _ptr(seq_lens), _ptr(w_uk), _ptr(w_uv), _ptr(out), _ptr(lse),
                                              _stream_handle())
    _check(st, "da_mla_decode_absorbed_noalloc")
    return out, lse


def _mla_paged_params(q_nope, q_rope, cache_pool, w_uv, max_seq_len, softmax_scale,
                      num_splits) -> MlaParams:
    # the params describe a [B, max_seq_len, 576] cache with the pool's token
    # stride (the batch stride is unused for paged pools)
    p = mla_params(q_nope, cache_pool[:1].expand(q_nope.shape[0], -1, -1), w_uv, q_rope,
                   softmax_scale, num_splits)
    p.max_seq_len = int(max_seq_len)
    p.cache_stride_b = 0
    return p


def mla_decode_absorbed_paged(q_nope: torch.Tensor, q_rope: torch.Tensor, cache_pool: torch.Tensor,
                              block_table: torch.Tensor, page_size: int, seq_lens: torch.Tensor,
                              w_uk: torch.Tensor, w_uv: torch.Tensor,
                              max_seq_len: Optional[int] = None,
                              softmax_scale: Optional[float] = None,
                              num_splits: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_decode_absorbed over a paged latent pool cache_pool [num_pages,
    page_size, 576] bf16 and block_table [B, max_blocks_per_seq] int32."""
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("cache_pool", cache_pool),
                    ("w_uk", w_uk), ("w_uv", w_uv)):
        _require_cuda(name, t)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("w_uk", w_uk), ("w_uv", w_uv)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, _ = q_nope.shape
    _check_seq_lens(seq_lens, B)
    if block_table.shape[0] != B:
        raise ValueError("block_table must have one row per sequence")
    pg = paged_kv(block_table, page_size, cache_pool)
    if max_seq_len is None:
        max_seq_len = block_table.shape[1] * page_size
    p = _mla_paged_params(q_nope, q_rope, cache_pool, w_uv, max_seq_len, softmax_scale,
                          num_splits)
    L = lib()
    out = torch.empty((B, H, w_uv.shape[2]), dtype=torch.float32, device=q_nope.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device)
    ws_bytes = L.da_mla_decode_workspace_size(ctypes.byref(p))
    ws = _workspace(ws_bytes, q_nope.device)
    st = L.da_mla_decode_absorbed_paged(ctypes.byref(p), ctypes.byref(pg), _ptr(q_nope),
                                        _ptr(q_rope), _ptr(cache_pool), _ptr(seq_lens), _ptr(w_uk),
                                        _ptr(w_uv), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                        _stream_handle())
    _check(st, "da_mla_decode_absorbed_paged")
    return out, lse


def mla_stages(q_nope, q_rope, kv_cache, w_uk, w_uv, seq_lens=None, softmax_scale=None,
               num_splits: int = 0, paged: Optional[Tuple[torch.Tensor, int, int]] = None):
    """The three stages of mla_decode_absorbed as separate callables sharing
    buffers: returns (absorb, attend, merge, out, lse, buffers). Calling
    absorb(); attend(); merge() in order on one stream fills out and lse exactly
    as mla_decode_absorbed does. paged = (block_table, page_size, max_seq_len)
    makes kv_cache a paged pool [num_pages, page_size, 576] and the attend
    stage da_mla_attend_split_pass_paged."""
    pg = None
    if paged is not None:
        table, page_size, max_seq_len = paged
        pg = paged_kv(table, page_size, kv_cache)
        p = _mla_paged_params(q_nope, q_rope, kv_cache, w_uv, max_seq_len, softmax_scale,
                              num_splits)
    else:
        p = mla_params(q_nope, kv_cache, w_uv, q_rope, softmax_scale, num_splits)
    L = lib()
    po_bytes, pl_bytes = ctypes.c_size_t(), ctypes.c_size_t()
    _check(L.da_mla_partials_size(ctypes.byref(p), ctypes.byref(po_bytes), ctypes.byref(pl_bytes)),
           "da_mla_partials_size")
    B, H, _ = q_nope.shape
    dev = q_nope.device
    # absorbed queries [B, H, 576], then the low parts of q~ [B, H, 512]
    d_c = w_uv.shape[1]
    q_hat = torch.empty((B * H * (kv_cache.shape[2] + d_c),), dtype=torch.bfloat16, device=dev)
    # opaque partial buffers (slots of o~_s and lse_s; the library's layout)
    part_out = torch.empty((po_bytes.value,), dtype=torch.uint8, device=dev)
    part_lse = torch.empty((pl_bytes.value // 4,), dtype=torch.float32, device=dev)
    out = torch.empty((B, H, w_uv.shape[2]), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)

    def absorb():
        _check(L.da_mla_absorb_query(ctypes.byref(p), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                     _ptr(q_hat), _stream_handle()), "da_mla_absorb_query")

    def attend():
        if pg is None:
            _check(L.da_mla_attend_split_pass(ctypes.byref(p), _ptr(q_hat), _ptr(kv_cache),
                                              _ptr(seq_lens), _ptr(part_out), _ptr(part_lse),
                                              _stream_handle()), "da_mla_attend_split_pass")
        else:
            _check(L.da_mla_attend_split_pass_paged(ctypes.byref(p), ctypes.byref(pg), _ptr(q_hat),
                                                    _ptr(kv_cache), _ptr(seq_lens), _ptr(part_out),
                                                    _ptr(part_lse), _stream_handle()),
                   "da_mla_attend_split_pass_paged")

    def merge():
        _check(L.da_mla_merge_project(ctypes.byref(p), _ptr(q_hat), _ptr(part_out), _ptr(part_lse),
                                      _ptr(w_uv), _ptr(out), _ptr(lse), _stream_handle()),
               "da_mla_merge_project")

    return absorb, attend, merge, out, lse, dict(q_hat=q_hat, part_out=part_out, part_lse=part_lse)


def mla_num_splits(q_nope, q_rope, kv_cache, w_uv, num_splits: int = 0) -> int:
    """Fixed split count per sequence, or 0 when the splits are balanced on the
    device from the sequence lengths."""
    p = mla_params(q_nope, kv_cache, w_uv, q_rope, None, num_splits)
    return int(lib().da_mla_decode_num_splits(ctypes.byref(p)))


# ----------------------------------------------------------------------------
# split-KV merge
# ----------------------------------------------------------------------------

def splitkv_combine(partial_out: torch.Tensor, partial_lse: torch.Tensor,
                    out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge split partials: partial_out [S,B,H,D], partial_lse [S,B,H] (float32)."""
    _require_cuda("partial_out", partial_out)
    _require_cuda("partial_lse", partial_lse)
    if partial_out.dtype != torch.float32 or partial_lse.dtype != torch.float32:
        raise ValueError("partials must be float32")
    if not partial_out.is_contiguous() or not partial_lse.is_contiguous():
        raise ValueError("partials must be contiguous")
    S, B, H, D = partial_out.shape
    if partial_lse.shape != (S, B, H):
        raise ValueError("partial_lse must be [S, B, H]")
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=partial_out.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=partial_out.device)
    st = lib().da_splitkv_combine(S, B, H, D, _ptr(partial_out), _ptr(partial_lse), _ptr(out),
                                  _ptr(lse), _stream_handle())
    _check(st, "da_splitkv_combine")
    return out, lse


__all__ = ["gqa_decode", "mla_decode_absorbed", "splitkv_combine", "gqa_num_splits",
           "mla_num_splits", "gqa_decode_paged", "mla_decode_absorbed_paged", "paged_kv",
           "gqa_decode_fp8", "KvScales", "lib",
           "LIB_PATH", "GqaParams", "MlaParams", "PagedKv", "DecodeAttnError", "LibraryMissing"]


# ----------------------------------------------------------------------------
# cache append with rotary position embedding
# ----------------------------------------------------------------------------

def _append_desc(rotary_dim: int, style: str, base: float, inv_freq: Optional[torch.Tensor],
                 new_stride_b: int, new_stride_h: int) -> Append:
    if style not in ROPE_STYLES:
        raise ValueError(f"style must be one of {sorted(ROPE_STYLES)}")
    ap = Append()
    ap.rotary_dim, ap.rope_style, ap.rope_base = int(rotary_dim), ROPE_STYLES[style], float(base)
    if inv_freq is not None:
        _require_cuda("inv_freq", inv_freq)
        if inv_freq.dtype != torch.float32 or inv_freq.shape != (rotary_dim // 2,) or \
                not inv_freq.is_contiguous():
            raise ValueError("inv_freq must be a contiguous float32 tensor of shape [rotary_dim / 2]")
        ap.inv_freq = inv_freq.data_ptr()
    ap.new_stride_b, ap.new_stride_h = int(new_stride_b), int(new_stride_h)
    return ap


def _check_positions(positions: torch.Tensor, B: int):
    _require_cuda("positions", positions)
    if positions.dtype != torch.int32 or positions.shape != (B,) or not positions.is_contiguous():
        raise ValueError("positions must be a contiguous int32 tensor of shape [B]")


def gqa_append_rope(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                    positions: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    rotary_dim: Optional[int] = None, style: str = "half", base: float = 10000.0,
                    inv_freq: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None,
                    block_table: Optional[torch.Tensor] = None, page_size: int = 0,
                    max_seq_len: Optional[int] = None) -> torch.Tensor:
    """Append one token per sequence to a GQA cache, rotating q and the new key.

    q [B, Hq, D]; k_new, v_new [B, Hkv, D] (same strides); positions [B] int32
    (row written and rotation position; outside [0, L_max) skips the
    sequence). k_cache, v_cache [B, L_max, Hkv, D], or paged pools
    [num_pages, page_size, Hkv, D] with block_table [B, max_blocks] int32.
    Returns q_out (the rotated queries; pass q_out=q to rotate in place).
    rotary_dim defaults to D; style "half" pairs (i, i + r/2), "interleaved"
    (2i, 2i + 1); inv_freq [r/2] float32 overrides base^(-2i/r)."""
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        _require_cuda(name, t)
    if len({t.dtype for t in (q, k_new, v_new, k_cache, v_cache)}) != 1:
        raise ValueError("q, k_new, v_new and the caches must share a dtype")
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("v_cache must have the shape and strides of k_cache")
    B, Hq, D = q.shape
    if k_new.shape != (B, k_cache.shape[2], D) or v_new.shape != k_new.shape or \
            v_new.stride() != k_new.stride() or k_new.stride(2) != 1:
        raise ValueError("k_new and v_new must be [B, Hkv, D] with one stride set and a contiguous D axis")
    _check_positions(positions, B)
    if q_out is None:   # the C ABI writes q_out in q's strides
        q_out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if q_out.shape != q.shape or q_out.stride() != q.stride() or q_out.dtype != q.dtype:
        raise ValueError("q_out must match q in shape, strides and dtype")
    pg = None
    if block_table is not None:
        pg = paged_kv(block_table, page_size, k_cache)
        if block_table.shape[0] != B:
            raise ValueError("block_table must have one row per sequence")
        L_max = block_table.shape[1] * page_size if max_seq_len is None else int(max_seq_len)
        p = gqa_params(q, k_cache[:1].expand(B, -1, -1, -1), None, 0)
        p.max_seq_len, p.kv_stride_b = L_max, 0
    else:
        p = gqa_params(q, k_cache, None, 0)
    ap = _append_desc(D if rotary_dim is None else rotary_dim, style, base, inv_freq,
                      k_new.stride(0), k_new.stride(1))
    st = _call("da_gqa_append_rope", ctypes.byref(p), ctypes.byref(ap),
                                  None if pg is None else ctypes.byref(pg), _ptr(q), _ptr(q_out),
                                  _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(k_cache),
                                  _ptr(v_cache), _stream_handle())
    _check(st, "da_gqa_append_rope")
    return q_out


def gqa_append_rope_fp8(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        positions: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        k_scale: torch.Tensor, v_scale: torch.Tensor,
                        rotary_dim: Optional[int] = None, style: str = "half", base: float = 10000.0,
                        inv_freq: Optional[torch.Tensor] = None,
                        q_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gqa_append_rope into an E4M3 cache: q, k_new, v_new bf16; k_cache,
    v_cache uint8 codes [B, L_max, Hkv, D]; k_scale, v_scale float32
    [B, L_max, Hkv]. With a nonzero token stride the appended rows' scales are computed
    (max|x| / 448) and written; with a zero token stride (broadcast per-head
    scales) they are read. Returns q_out."""
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache), ("k_scale", k_scale), ("v_scale", v_scale)):
        _require_cuda(name, t)
    if any(t.dtype != torch.bfloat16 for t in (q, k_new, v_new)):
        raise ValueError("q, k_new and v_new must be bfloat16")
    if k_cache.dtype == torch.float8_e4m3fn:
        k_cache, v_cache = k_cache.view(torch.uint8), v_cache.view(torch.uint8)
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("k_cache and v_cache must hold E4M3 codes (uint8 or float8_e4m3fn)")
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("v_cache must have the shape and strides of k_cache")
    if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32 or \
            k_scale.stride() != v_scale.stride() or k_scale.dim() != 3:
        raise ValueError("k_scale and v_scale must be float32 [B, L_max, Hkv] with one stride set")
    B, Hq, D = q.shape
    if k_new.shape != (B, k_cache.shape[2], D) or v_new.shape != k_new.shape or \
            v_new.stride() != k_new.stride() or k_new.stride(2) != 1:
        raise ValueError("k_new and v_new must be [B, Hkv, D] with one stride set and a contiguous D axis")
    if k_cache.shape[0] != B or k_cache.stride(3) != 1 or \
            k_scale.shape != (B, k_cache.shape[1], k_cache.shape[2]) or v_scale.shape != k_scale.shape:
        raise ValueError("k_cache must be [B, L_max, Hkv, D] (contiguous D) and the scales [B, L_max, Hkv]")
    _check_positions(positions, B)
    if q_out is None:
        q_out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if q_out.shape != q.shape or q_out.stride() != q.stride() or q_out.dtype != q.dtype:
        raise ValueError("q_out must match q in shape, strides and dtype")
    p = GqaParams()
    p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim = B, Hq, k_cache.shape[2], D
    p.dtype = DA_DTYPE_FP8_E4M3
    p.softmax_scale = 1.0 / math.sqrt(D)
    p.q_stride_b, p.q_stride_h = q.stride(0), q.stride(1)
    p.kv_stride_t, p.kv_stride_h = k_cache.stride(1), k_cache.stride(2)
    p.max_seq_len, p.kv_stride_b = k_cache.shape[1], k_cache.stride(0)
    sc = KvScales()
    sc.k_scale, sc.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
    sc.stride_b, sc.stride_t, sc.stride_h = k_scale.stride()
    ap = _append_desc(D if rotary_dim is None else rotary_dim, style, base, inv_freq,
                      k_new.stride(0), k_new.stride(1))
    st = _call("da_gqa_append_rope_fp8", ctypes.byref(p), ctypes.byref(ap), None,
               ctypes.byref(sc), _ptr(q), _ptr(q_out),
               _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(k_cache), _ptr(v_cache),
               _stream_handle())
    _check(st, "da_gqa_append_rope_fp8")
    return q_out


def mla_append_rope(q_rope: torch.Tensor, kv_new: torch.Tensor, positions: torch.Tensor,
                    kv_cache: torch.Tensor, rotary_dim: int = 64, style: str = "half",
                    base: float = 10000.0, inv_freq: Optional[torch.Tensor] = None,
                    q_rope_out: Optional[torch.Tensor] = None,
                    block_table: Optional[torch.Tensor] = None, page_size: int = 0,
                    max_seq_len: Optional[int] = None) -> torch.Tensor:
    """Append one latent row per sequence to an MLA cache: row positions[b]
    becomes [kv_new[b, :512] ; RoPE(kv_new[b, 512:])], and the query rope
    parts q_rope [B, H, 64] are rotated. kv_new [B, 576] bf16 (row-contiguous);
    kv_cache [B, L_max, 576] bf16, or a paged pool [num_pages, page_size, 576]
    with block_table. Returns q_rope_out (q_rope_out=q_rope rotates in place)."""
    for name, t in (("q_rope", q_rope), ("kv_new", kv_new), ("kv_cache", kv_cache)):
        _require_cuda(name, t)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    B, H, d_rope = q_rope.shape
    if not q_rope.is_contiguous() or kv_new.dim() != 2 or kv_new.shape[0] != B or \
            kv_new.shape[1] != kv_cache.shape[-1] or kv_new.stride(1) != 1:
        raise ValueError("q_rope must be contiguous [B, H, 64] and kv_new [B, 576] with contiguous rows")
    _check_positions(positions, B)
    if q_rope_out is None:
        q_rope_out = torch.empty_like(q_rope)
    if q_rope_out.shape != q_rope.shape or not q_rope_out.is_contiguous() or q_rope_out.dtype != q_rope.dtype:
        raise ValueError("q_rope_out must be a contiguous bf16 tensor shaped like q_rope")
    d_c = kv_cache.shape[-1] - d_rope
    # the params only carry shapes here; W_UV's shape is fixed by the format
    fake_uv = torch.empty((H, d_c, 128), dtype=torch.bfloat16, device="meta")
    q_nope = torch.empty((B, H, 128), dtype=torch.bfloat16, device="meta")
    pg = None
    if block_table is not None:
        pg = paged_kv(block_table, page_size, kv_cache)
        if block_table.shape[0] != B:
            raise ValueError("block_table must have one row per sequence")
        L_max = block_table.shape[1] * page_size if max_seq_len is None else int(max_seq_len)
        p = _mla_paged_params(q_nope, q_rope, kv_cache, fake_uv, L_max, None, 0)
    else:
        p = mla_params(q_nope, kv_cache, fake_uv, q_rope, None, 0)
    ap = _append_desc(rotary_dim, style, base, inv_freq, kv_new.stride(0), 0)
    st = _call("da_mla_append_rope", ctypes.byref(p), ctypes.byref(ap),
                                  None if pg is None else ctypes.byref(pg), _ptr(q_rope),
                                  _ptr(q_rope_out), _ptr(kv_new), _ptr(positions), _ptr(kv_cache),
                                  _stream_handle())
    _check(st, "da_mla_append_rope")
    return q_rope_out


# ----------------------------------------------------------------------------
# streaming probes (bandwidth ceiling; not part of the attention path)
# ----------------------------------------------------------------------------

def _probe_buffer(name: str, t: torch.Tensor):
    _require_cuda(name, t)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def probe_stream_read(src: torch.Tensor, sink: torch.Tensor, blocks: int = 0, depth: int = 8) -> None:
    """Read every byte of `src` once; XOR the XOR of its 32-bit words into
    sink[0] (an int32 device tensor the caller clears). blocks = workgroups
    (0: one per compute unit); depth = 16-byte loads in flight per thread."""
    _probe_buffer("src", src)
    _require_cuda("sink", sink)
    if sink.dtype != torch.int32 or sink.numel() < 1:
        raise ValueError("sink must be an int32 tensor with at least one element")
    nbytes = src.numel() * src.element_size()
    _check(_call("da_probe_stream_read", _ptr(src), nbytes, blocks, depth, _ptr(sink),
                 _stream_handle()), "da_probe_stream_read")


def probe_stream_copy(src: torch.Tensor, dst: torch.Tensor, blocks: int = 0, depth: int = 4) -> None:
    """Copy the bytes of `src` into `dst` (same byte size, no overlap)."""
    _probe_buffer("src", src)
    _probe_buffer("dst", dst)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same byte size")
    _check(_call("da_probe_stream_copy", _ptr(src), _ptr(dst), nbytes, blocks, depth,
                 _stream_handle()), "da_probe_stream_copy")
