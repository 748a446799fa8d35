"""Helpers for the GPU parity tests: host arrays -> device tensors, and the
comparison bar.

The bar for floating-point outputs (bf16 inputs, fp32 accumulation):
  * output: per row (b, h), max_d |o - o_ref| / max_d |o_ref| <= 1e-2;
  * lse:    max |lse - lse_ref| <= 1e-3 (absolute, natural log).
Rows whose reference is empty (lse_ref = -inf) must come back exactly
out = 0 and lse = -inf.
"""
import os
import sys

import numpy as np
import torch

OUT_RTOL = 1e-2
LSE_ATOL = 1e-3

# Largest errors seen per parity check, keyed by test and check name; written
# to the file named by DA_PARITY_RECORD at the end of the session (conftest).
RECORD = {}


def _record(what, rel, lerr, out_rtol, lse_atol):
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    tol = np.asarray(out_rtol, dtype=np.float64)
    RECORD[f"{test} :: {what}"] = dict(max_row_rel_err=rel, max_lse_abs_err=lerr,
                                       out_rtol=float(tol.max()) if tol.size else None,
                                       lse_atol=float(lse_atol))


def announce(msg: str):
    """Print (and flush) which case is about to run on the GPU."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def f32_tensor(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def gqa_to_device(inp):
    conv = bf16_tensor if inp.dtype == "bf16" else f32_tensor
    return (conv(inp.q), conv(inp.k), conv(inp.v),
            torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda())


def mla_to_device(inp):
    return (bf16_tensor(inp.q_nope), bf16_tensor(inp.q_rope), bf16_tensor(inp.cache),
            bf16_tensor(inp.w_uk), bf16_tensor(inp.w_uv),
            torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda())


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> np.ndarray:
    err = np.abs(out.astype(np.float64) - ref).max(axis=-1)
    scale = np.abs(ref).max(axis=-1)
    return err / np.maximum(scale, 1e-30)


def assert_parity(out, lse, ref_out, ref_lse, out_rtol=OUT_RTOL, lse_atol=LSE_ATOL, what=""):
    """out/lse: numpy (from the GPU); ref_*: float64 oracle results."""
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    empty = np.isneginf(ref_lse)
    if empty.any():
        assert np.all(np.isneginf(lse[empty])), f"{what}: empty rows must give lse=-inf"
        assert np.all(out[empty] == 0), f"{what}: empty rows must give out=0"
    full = ~empty
    if not full.any():
        _record(what, 0.0, 0.0, out_rtol, lse_atol)
        return 0.0, 0.0
    assert np.isfinite(out[full]).all(), f"{what}: non-finite outputs"
    assert np.isfinite(lse[full]).all(), f"{what}: non-finite lse"
    rel = row_rel_err(out[full], ref_out[full])
    lerr = np.abs(lse[full] - ref_lse[full])
    _record(what, float(rel.max()), float(lerr.max()), out_rtol, lse_atol)
    tol = np.broadcast_to(np.asarray(out_rtol, dtype=np.float64), np.shape(ref_lse))[full]
    assert np.all(rel <= tol), f"{what}: row-relative output error {rel.max():.3e} over its bound"
    assert lerr.max() <= lse_atol, f"{what}: max lse error {lerr.max():.3e} > {lse_atol}"
    return float(rel.max()), float(lerr.max())


def bf16_weight_bound(q, k, v, seq_lens, scale, ref_out, ref_lse):
    """Per row (b, h) of a GQA decode: the output error that rounding each
    softmax weight to bf16 can cause, relative to the row's largest output,
    plus fp32 accumulation slack. bf16 keeps 8 significant bits, so rounding
    to nearest gives p~_j = p_j (1 + d_j) with |d_j| <= 2^-8, and o_d changes
    by at most 2^-8 sum_j p_j |v_jd|. q [B, Hq, D], k and v
    [B, L, Hkv, D] float64 (the values the kernel sees), ref_* from the oracle."""
    B, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    bound = np.zeros((B, Hq))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        for kv in range(Hkv):
            hs = slice(kv * g, (kv + 1) * g)
            s = scale * q[b, hs] @ k[b, :L, kv].T                        # [g, L]
            p = np.exp(s - ref_lse[b, hs, None])
            spread = (p @ np.abs(v[b, :L, kv])).max(axis=-1)             # [g]
            bound[b, hs] = 2.0 ** -8 * spread / np.maximum(np.abs(ref_out[b, hs]).max(axis=-1), 1e-30)
    return bound + 1e-5
