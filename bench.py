#!/usr/bin/env python3
"""Benchmark of single-token decode attention on one MI355X.

One step is one pass of the whole hot path on synthetic inputs:
  * GQA decode, Llama-3-8B shape: batch 32, 32 query / 8 KV heads, d_head 128,
    every sequence at 4096 cached rows, bf16 (split pass + log-sum-exp merge);
  * absorbed-MLA decode, DeepSeek-V3 shape: batch 64, 128 heads, latent cache
    [64, 4096, 576] bf16, W_UK / W_UV [128, 512, 128] (query absorption,
    split-KV latent attention, merge + W_UV projection).
Other workloads (--workload): each path alone, long-context MLA, ragged
MHA, GQA / MLA over paged caches (pools of 16-row pages in a seeded random
physical order, read through a block table), GQA over an FP8 (E4M3)
cache with one fp32 scale per (token, KV head) for K and for V, sliding-window
GQA (8192 cached rows, window 4096), and the step before decode: appending the
new token's rows with RoPE (bf16 GQA and MLA caches, `append`; an E4M3 GQA
cache, `append-fp8`). The append kernels take a few microseconds, less than
the Python binding's per-call checks, so those steps replay the recorded C
calls, and their roofline pass is queued behind a GPU spin so the launches
are issued ahead of the GPU.
Inputs are resident in HBM before timing starts. The default warm-up (200
steps, about 40 ms) outlasts the board's power-management transient: in a
kernel trace of this step, the first few milliseconds of back-to-back steps
run the attention kernels up to a third slower than the steady state they
reach after about 20 ms. Each step reads the next of
several copies of the caches, so that no step finds the previous step's cache
in the 256 MB last-level (Infinity) cache.

Prints ONE JSON line on stdout. `value` is algorithmic bytes per step (cache
rows once, queries, weights, outputs) over the wall time per step of the timed
region, in GB/s. The timed region has no event between launches: an event
makes the next kernel wait for the previous one to finish completely, so
consecutive kernels no longer overlap at their edges. An untimed probe pass
with an event between every two launches gives the per-kernel breakdown
(`paths`) and picks the dominant kernel; a roofline pass of K further steps,
with HIP events on the launch stream around every launch of that kernel, gives
its average duration for the `roofline` object. Timing events are created
without the system-scope fence of default events (which writes back and
invalidates the caches at every event). `cpu_baseline` times the fp64 CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn KV GB/s & TFLOP/s per layer-step; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
MALL_GUARD_BYTES = 1 << 30     # rotate through >= 1 GiB of distinct cache copies
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipTimingEvents:
    """HIP events for timing only, created with hipEventDisableSystemFence.

    A default event performs a system-scope release when it is reached, which
    writes back and invalidates the GPU caches; on MI355X that costs the
    stream several microseconds per event and slows the kernel after it. These
    events skip the fence (their elapsed times are still ordered by the
    stream). They bind to the HIP runtime torch has already loaded (same
    soname), and are recorded on the stream the library's launches go to."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        import torch  # noqa: F401  (loads the process's HIP runtime first)
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        vp = ctypes.c_void_p
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [vp, vp]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        self.hip.hipEventDestroy.argtypes = [vp]
        self.events = []

    def create(self):
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.events.append(ev)
        return ev

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ev, self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


class Telemetry:
    """Samples the GPU's current shader clock (the active level of
    pp_dpm_sclk) and board power (hwmon power1_input) from sysfs every
    ~20 ms in a background thread while a region runs. Reports medians;
    an empty result where the files are not readable."""

    def __init__(self):
        import glob
        self.sclk_path = self.power_path = None
        for card in sorted(glob.glob("/sys/class/drm/card*/device")):
            p = os.path.join(card, "pp_dpm_sclk")
            if self.sclk_path is None and os.path.exists(p):
                self.sclk_path = p
                hw = sorted(glob.glob(os.path.join(card, "hwmon", "hwmon*", "power1_input")))
                self.power_path = hw[0] if hw else None
        self.samples = []

    def _read(self):
        rec = {}
        try:
            if self.sclk_path:
                for line in open(self.sclk_path).read().splitlines():
                    if line.strip().endswith("*"):
                        rec["sclk_mhz"] = float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
            if self.power_path:
                rec["power_w"] = int(open(self.power_path).read().strip()) / 1e6
        except (OSError, ValueError, IndexError):
            pass
        return rec

    def __enter__(self):
        import threading
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                r = self._read()
                if r:
                    self.samples.append(r)
                self._stop.wait(0.02)
        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self):
        out = {"samples": len(self.samples)}
        for k in ("sclk_mhz", "power_w"):
            v = [r[k] for r in self.samples if k in r]
            if v:
                out[k + "_median"] = round(float(np.median(v)), 1)
        return out


def rocm_version():
    for path in ("/opt/rocm/.info/version",):
        try:
            return open(path).read().strip()
        except OSError:
            pass
    try:
        import torch
        return f"hip {torch.version.hip}"
    except Exception:  # pragma: no cover
        return "unknown"


# ----------------------------------------------------------------------------
# algorithmic traffic and work (what the method must move / compute)
# ----------------------------------------------------------------------------

def gqa_alg(B, Hq, Hkv, D, total_rows, elem=2):
    """Bytes: every cached K and V row once, q, fp32 out + lse. FLOPs: 2 per
    dimension for q.k and for p.v, per query head and cached row."""
    cache = total_rows * 2 * Hkv * D * elem
    q = B * Hq * D * elem
    out = B * Hq * (D + 1) * 4
    return dict(cache=cache, q=q, out=out, total=cache + q + out, flops=4 * Hq * D * total_rows)


def mla_alg(B, H, total_rows, d_c=512, d_r=64, d_n=128, d_v=128, elem=2):
    """Bytes: every cached latent row (576 elements of `elem` bytes) once,
    W_UK and W_UV once, q_nope/q_rope, fp32 out + lse. FLOPs: per cached row
    2*H*(576 + 512), plus the two per-head projections 2*B*H*d_c*(d_n + d_v)."""
    cache = total_rows * (d_c + d_r) * elem
    weights = 2 * H * d_c * 128 * 2
    q = B * H * (d_n + d_r) * 2
    out = B * H * (d_v + 1) * 4
    attn_flops = H * 2 * ((d_c + d_r) + d_c) * total_rows
    proj_flops = 2 * B * H * d_c * (d_n + d_v)
    return dict(cache=cache, weights=weights, q=q, out=out, total=cache + weights + q + out,
                flops=attn_flops + proj_flops, attn_flops=attn_flops)


# ----------------------------------------------------------------------------
# GPU part
# ----------------------------------------------------------------------------

def to_dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def setup_gqa(cfg):
    import torch
    import workloads as W
    import decode_attention_kv_bf16_amd as da
    inp = W.make_gqa_config(cfg)
    q = to_dev_bf16(inp.q)
    k0, v0 = to_dev_bf16(inp.k), to_dev_bf16(inp.v)
    sl = torch.from_numpy(inp.seq_lens).cuda()
    fp = k0.numel() * 2 * 2
    n_copies = max(1, math.ceil(MALL_GUARD_BYTES / fp)) if fp < MALL_GUARD_BYTES else 1
    copies = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(n_copies - 1)]
    S = da.gqa_num_splits(q, k0)
    B, Hq, D = q.shape
    part_out = torch.empty((S, B, Hq, D), dtype=torch.float32, device="cuda")
    part_lse = torch.empty((S, B, Hq), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    calls = []
    for kk, vv in copies:
        def split_pass(kk=kk, vv=vv):
            da.gqa_decode_split_pass(q, kk, vv, sl, inp.scale, part_out=part_out, part_lse=part_lse)

        def combine():
            da.splitkv_combine(part_out, part_lse, out=out, lse=lse)
        # with one split the pass writes the final output itself
        calls.append([("gqa_split_pass", split_pass)] + ([("gqa_combine", combine)] if S > 1 else []))
    alg = gqa_alg(B, Hq, k0.shape[2], D, int(inp.seq_lens.sum()))
    info = dict(batch=B, q_heads=Hq, kv_heads=int(k0.shape[2]), head_dim=D,
                seq_len=int(inp.seq_lens.max()), splits=S, cache_copies=len(copies))
    return calls, alg, info, inp


WINDOW = 4096          # Mistral 7B's sliding window ("Attention variants and KV cache", section 5.3)
WINDOW_CONTEXT = 8192  # rows per sequence in the cache; only the last WINDOW are attended


def setup_gqa_window():
    """Sliding-window GQA decode: the Llama-3-8B GQA shape (Mistral 7B has the same
    32 query heads, 8 KV heads and d 128) with 8192 cached rows per sequence
    and a 4096-row window, so each call reads the same bytes as the 4096-row call without a window."""
    import torch
    import workloads as W
    import decode_attention_kv_bf16_amd as da
    inp = W.make_gqa(32, 32, 8, 128, [WINDOW_CONTEXT] * 32, cfg=2)
    q = to_dev_bf16(inp.q)
    k, v = to_dev_bf16(inp.k), to_dev_bf16(inp.v)
    sl = torch.from_numpy(inp.seq_lens).cuda()
    B, Hq, D = q.shape
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

    def call():
        da.gqa_decode(q, k, v, sl, inp.scale, out=out, lse=lse, window=WINDOW)
    rows = int(np.minimum(inp.seq_lens, WINDOW).sum())
    alg = gqa_alg(B, Hq, k.shape[2], D, rows)
    info = dict(batch=B, q_heads=Hq, kv_heads=int(k.shape[2]), head_dim=D, seq_len=WINDOW_CONTEXT,
                window=WINDOW, splits=da.gqa_num_splits(q, k, window=WINDOW))
    return [[("gqa_window", call)]], alg, info, inp


def setup_mla(cfg):
    import torch
    import workloads as W
    import decode_attention_kv_bf16_amd as da
    inp = W.make_mla_config(cfg)
    qn, qr = to_dev_bf16(inp.q_nope), to_dev_bf16(inp.q_rope)
    wuk, wuv = to_dev_bf16(inp.w_uk), to_dev_bf16(inp.w_uv)
    c0 = to_dev_bf16(inp.cache)
    sl = torch.from_numpy(inp.seq_lens).cuda()
    fp = c0.numel() * 2
    n_copies = max(1, math.ceil(MALL_GUARD_BYTES / fp)) if fp < MALL_GUARD_BYTES else 1
    caches = [c0] + [c0.clone() for _ in range(n_copies - 1)]
    calls = []
    S = None
    for c in caches:
        absorb, attend, merge, _, _, bufs = da.mla_stages(qn, qr, c, wuk, wuv, sl, inp.scale)
        S = da.mla_num_splits(qn, qr, c, wuv) or "balanced"
        calls.append([("mla_absorb", absorb), ("mla_attend", attend), ("mla_merge_project", merge)])
    B, H, _ = qn.shape
    alg = mla_alg(B, H, int(inp.seq_lens.sum()))
    info = dict(batch=B, heads=H, seq_len=int(inp.seq_lens.max()),
                total_rows=int(inp.seq_lens.sum()), splits=S, cache_copies=len(caches))
    return calls, alg, info, inp


def setup_mla_fp8(cfg):
    """The MLA workload of `cfg` with the latent cache in E4M3 and two fp32
    scales per (sequence, token), one for the c_kv range and one for the
    k_rope range; one call of the whole decode per step."""
    import torch
    import workloads as W
    import decode_attention_kv_bf16_amd as da
    inp = W.make_mla_fp8_config(cfg)
    qn, qr = to_dev_bf16(inp.q_nope), to_dev_bf16(inp.q_rope)
    wuk, wuv = to_dev_bf16(inp.w_uk), to_dev_bf16(inp.w_uv)
    c0 = torch.from_numpy(inp.cache).cuda()
    sn, sr = torch.from_numpy(inp.scale_nope).cuda(), torch.from_numpy(inp.scale_rope).cuda()
    sl = torch.from_numpy(inp.seq_lens).cuda()
    fp = c0.numel()
    n_copies = max(1, math.ceil(MALL_GUARD_BYTES / fp)) if fp < MALL_GUARD_BYTES else 1
    caches = [c0] + [c0.clone() for _ in range(n_copies - 1)]
    B, H, _ = qn.shape
    out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    calls = []
    for c in caches:
        def call(c=c):
            da.mla_decode_absorbed_fp8(qn, qr, c, sn, sr, wuk, wuv, sl, inp.scale, out=out, lse=lse)
        calls.append([("mla_decode_fp8", call)])
    rows = int(inp.seq_lens.sum())
    alg = mla_alg(B, H, rows, elem=1)
    scale_bytes = 2 * rows * 4
    alg["cache"] += scale_bytes
    alg["total"] += scale_bytes
    info = dict(batch=B, heads=H, seq_len=int(inp.seq_lens.max()), total_rows=rows,
                cache="e4m3 + fp32 c_kv and k_rope scales per (sequence, token)", cache_copies=len(caches))
    return calls, alg, info, inp


def setup_mla_fp8_paged(cfg):
    """The E4M3 MLA workload of `cfg` with the codes and both scale arrays in
    pools of 16-row pages (one block table)."""
    import torch
    import workloads as W
    import decode_attention_kv_bf16_amd as da
    inp = W.make_mla_fp8_config(cfg)
    (cp_h, snp_h, srp_h), table_h = paged_pools(inp.seq_lens, [inp.cache, inp.scale_nope, inp.scale_rope],
                                                seed=cfg)
    qn, qr = to_dev_bf16(inp.q_nope), to_dev_bf16(inp.q_rope)
    wuk, wuv = to_dev_bf16(inp.w_uk), to_dev_bf16(inp.w_uv)
    c0 = torch.from_numpy(cp_h).cuda()
    snp, srp = torch.from_numpy(snp_h).cuda(), torch.from_numpy(srp_h).cuda()
    table = torch.from_numpy(table_h).cuda()
    sl = torch.from_numpy(inp.seq_lens).cuda()
    fp = c0.numel()
    n_copies = max(1, math.ceil(MALL_GUARD_BYTES / fp)) if fp < MALL_GUARD_BYTES else 1
    pools = [c0] + [c0.clone() for _ in range(n_copies - 1)]
    B, H, _ = qn.shape
    L = inp.cache.shape[1]
    out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    calls = []
    for pl in pools:
        def call(pl=pl):
            da.mla_decode_absorbed_fp8_paged(qn, qr, pl, snp, srp, table, PAGE_SIZE, sl, wuk, wuv, max_seq_len=L,
                                             softmax_scale=inp.scale, out=out, lse=lse)
        calls.append([("mla_decode_fp8_paged", call)])
    rows = int(inp.seq_lens.sum())
    alg = mla_alg(B, H, rows, elem=1)
    extra = 2 * rows * 4 + table_h.nbytes
    alg["cache"] += 2 * rows * 4
    alg["total"] += extra
    info = dict(batch=B, heads=H, seq_len=int(inp.seq_lens.max()), total_rows=rows, page_size=PAGE_SIZE,
                num_pages=int(cp_h.shape[0]), cache="e4m3 + fp32 c_kv and k_rope scales, paged",
                cache_copies=len(pools))
    return calls, alg, info, (inp, dict(pools=(cp_h, snp_h, srp_h), table=table_h))


def binding_roofline(alg, t_ms):
    """Which roofline binds a whole call (the larger of its HBM time and its
    bf16 matrix-core time at peak) and the fraction of it reached."""
    hbm_ms = alg["total"] / (HBM_PEAK_GBS * 1e9) * 1e3
    mfma_ms = alg["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
    bound = "mfma" if mfma_ms > hbm_ms else "hbm"
    return dict(bound=bound, frac=round(max(hbm_ms, mfma_ms) / t_ms, 4))


PAGE_SIZE = 16   # rows per page of the paged workloads (the common default)


def paged_pools(seq_lens, caches, seed):
    """Host pools [num_pages, PAGE_SIZE, ...] of the given contiguous caches,
    pages in a seeded random physical order, and the block table."""
    import workloads as W
    table, n_pages = W.make_block_table(seq_lens, PAGE_SIZE, seed=seed, spare_pages=0)
    return [W.paginate(c, seq_lens, table, n_pages, PAGE_SIZE, 0) for c in caches], table


def setup_gqa_paged(cfg):
    """The GQA workload of `cfg` with K and V in pools of 16-row pages."""
    import torch
    import workloads as W
    import decode_attention_kv_bf16_amd as da
    inp = W.make_gqa_config(cfg)
    (kp_h, vp_h), table_h = paged_pools(inp.seq_lens, [inp.k, inp.v], seed=cfg)
    q = to_dev_bf16(inp.q)
    k0, v0 = to_dev_bf16(kp_h), to_dev_bf16(vp_h)
    table = torch.from_numpy(table_h).cuda()
    sl = torch.from_numpy(inp.seq_lens).cuda()
    fp = k0.numel() * 2 * 2
    n_copies = max(1, math.ceil(MALL_GUARD_BYTES / fp)) if fp < MALL_GUARD_BYTES else 1
    copies = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(n_copies - 1)]
    B, Hq, D = q.shape
    L = inp.k.shape[1]
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    calls = []
    for kk, vv in copies:
        def call(kk=kk, vv=vv):
            da.gqa_decode_paged(q, kk, vv, table, PAGE_SIZE, sl, max_seq_len=L,
                                softmax_scale=inp.scale, out=out, lse=lse)
        calls.append([("gqa_decode_paged", call)])
    alg = gqa_alg(B, Hq, inp.k.shape[2], D, int(inp.seq_lens.sum()))
    alg["total"] += table_h.nbytes
    info = dict(batch=B, q_heads=Hq, kv_heads=int(inp.k.shape[2]), head_dim=D,
                seq_len=int(inp.seq_lens.max()), page_size=PAGE_SIZE,
                num_pages=int(kp_h.shape[0]), cache_copies=len(copies))
    return calls, alg, info, (inp, dict(k_pool=kp_h, v_pool=vp_h, table=table_h))


def setup_mla_paged(cfg):
    """The MLA workload of `cfg` with the latent cache in a pool of 16-row pages."""
    import torch
    import workloads as W
    import decode_attention_kv_bf16_amd as da
    inp = W.make_mla_config(cfg)
    (pool_h,), table_h = paged_pools(inp.seq_lens, [inp.cache], seed=cfg)
    qn, qr = to_dev_bf16(inp.q_nope), to_dev_bf16(inp.q_rope)
    wuk, wuv = to_dev_bf16(inp.w_uk), to_dev_bf16(inp.w_uv)
    p0 = to_dev_bf16(pool_h)
    table = torch.from_numpy(table_h).cuda()
    sl = torch.from_numpy(inp.seq_lens).cuda()
    fp = p0.numel() * 2
    n_copies = max(1, math.ceil(MALL_GUARD_BYTES / fp)) if fp < MALL_GUARD_BYTES else 1
    pools = [p0] + [p0.clone() for _ in range(n_copies - 1)]
    L = inp.cache.shape[1]
    calls = []
    for pl in pools:
        absorb, attend, merge, _, _, _ = da.mla_stages(qn, qr, pl, wuk, wuv, sl, inp.scale,
                                                       paged=(table, PAGE_SIZE, L))
        calls.append([("mla_absorb", absorb), ("mla_attend_paged", attend),
                      ("mla_merge_project", merge)])
    B, H, _ = qn.shape
    alg = mla_alg(B, H, int(inp.seq_lens.sum()))
    alg["total"] += table_h.nbytes
    info = dict(batch=B, heads=H, seq_len=int(inp.seq_lens.max()),
                total_rows=int(inp.seq_lens.sum()), page_size=PAGE_SIZE,
                num_pages=int(pool_h.shape[0]), cache_copies=len(pools))
    return calls, alg, info, (inp, dict(pool=pool_h, table=table_h))


def head_major_codes(x):
    """E4M3 codes [X, T, H, D] (numpy) stored on the GPU head-major, [X, H, T,
    D], returned as the [X, T, H, D] view of that storage: each KV head's rows
    are then one contiguous run per sequence (or page)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).cuda()
    return t.permute(0, 2, 1, 3)


def clone_view(t):
    """A copy of `t` with the same strides (a permuted view's storage cloned)."""
    if t.is_contiguous():
        return t.clone()
    base = t.permute(0, 2, 1, 3)
    return base.clone().permute(0, 2, 1, 3)


def setup_gqa_fp8(cfg, layout="head"):
    """The GQA workload of `cfg` with K and V in E4M3 and one fp32 scale per
    (token, KV head) for each. layout "head": codes stored [B, Hkv, L, D]
    (each KV head's rows contiguous); "token": [B, L, Hkv, D] (a KV head's
    128-byte rows 1 KiB apart). Scales are token-major [B, L, Hkv] in both."""
    import torch
    import workloads as W
    import decode_attention_kv_bf16_amd as da
    inp = W.make_gqa_fp8_config(cfg)
    q = to_dev_bf16(inp.q)
    dev = lambda a: torch.from_numpy(a).cuda()
    # scales token-major [B, L, Hkv] (a KV head's scales 32 bytes apart): in
    # one process this layout measured 57.4 us per call against 68.4 us for
    # head-major scales with token-major codes, and 45.3 against 49.1 us with
    # head-major codes
    codes = head_major_codes if layout == "head" else dev
    k0, v0, ks, vs = codes(inp.k), codes(inp.v), dev(inp.k_scale), dev(inp.v_scale)
    sl = torch.from_numpy(inp.seq_lens).cuda()
    fp = k0.numel() * 2
    n_copies = max(1, math.ceil(MALL_GUARD_BYTES / fp)) if fp < MALL_GUARD_BYTES else 1
    copies = [(k0, v0)] + [(clone_view(k0), clone_view(v0)) for _ in range(n_copies - 1)]
    B, Hq, D = q.shape
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    calls = []
    for kk, vv in copies:
        def call(kk=kk, vv=vv):
            da.gqa_decode_fp8(q, kk, vv, ks, vs, sl, inp.scale, out=out, lse=lse)
        calls.append([("gqa_decode_fp8", call)])
    alg = gqa_alg(B, Hq, inp.k.shape[2], D, int(inp.seq_lens.sum()), elem=1)
    scale_bytes = 2 * int(inp.seq_lens.sum()) * inp.k.shape[2] * 4
    alg["cache"] += scale_bytes
    alg["total"] += scale_bytes
    info = dict(batch=B, q_heads=Hq, kv_heads=int(inp.k.shape[2]), head_dim=D,
                seq_len=int(inp.seq_lens.max()), cache="e4m3 + fp32 scale per (token, KV head)",
                codes="head-major [B, Hkv, L, D]" if layout == "head" else "token-major [B, L, Hkv, D]",
                cache_copies=len(copies))
    return calls, alg, info, inp


def replayed(wrapper_call):
    """Run a binding call once and return a function that repeats its C call
    with the same arguments. The append kernels take a few microseconds,
    less than the Python wrapper's argument checks, so the step replays the
    recorded call (the same launch) to keep the GPU, not Python, the limit."""
    import decode_attention_kv_bf16_amd as da
    with da.recorded_calls() as rec:
        wrapper_call()
    (fn, cargs), = rec

    def call():
        st = fn(*cargs)
        if st != 0:
            raise RuntimeError(f"{fn.__name__} failed with status {st}")
    return call


def setup_append(kind):
    """One token appended per sequence with RoPE: the Llama-3-8B GQA cache
    (B 32, Hq 32, Hkv 8, D 128, L 4096) or the DeepSeek-V3 MLA cache (B 64,
    H 128, rows of 576, L 4096), at seeded positions."""
    import torch
    import workloads as W
    import decode_attention_kv_bf16_amd as da
    if kind == "gqa-append":
        B, Hq, Hkv, D, L = 32, 32, 8, 128, 4096
        inp = W.make_gqa_append(B, Hq, Hkv, D, L, cfg=2)
        q, kn, vn = (to_dev_bf16(x) for x in (inp.q, inp.k_new, inp.v_new))
        kc = torch.zeros((B, L, Hkv, D), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        q_out = torch.empty_like(q)
        pos = torch.from_numpy(inp.positions).cuda()

        call = replayed(lambda: da.gqa_append_rope(q, kn, vn, pos, kc, vc, q_out=q_out))
        # bytes: q read and written, k and v rows read and written, positions;
        # FLOPs: 6 per rotated pair (q heads and the key heads)
        alg = dict(cache=2 * (2 * B * Hkv * D * 2), q=2 * B * Hq * D * 2, out=0,
                   flops=6 * B * (Hq + Hkv) * (D // 2))
        alg["total"] = alg["cache"] + alg["q"] + 4 * B
        info = dict(batch=B, q_heads=Hq, kv_heads=Hkv, head_dim=D, max_seq_len=L, rotary_dim=D,
                    rope="half pairs, base 10000")
        return [[("gqa_append_rope", call)]], alg, info, inp
    if kind == "gqa-append-fp8":
        # the Llama-3-8B GQA shape into an E4M3 cache with per-(token, KV head) scales
        # computed from the appended rows
        B, Hq, Hkv, D, L = 32, 32, 8, 128, 4096
        inp = W.make_gqa_append(B, Hq, Hkv, D, L, cfg=2)
        q, kn, vn = (to_dev_bf16(x) for x in (inp.q, inp.k_new, inp.v_new))
        kc = torch.zeros((B, L, Hkv, D), dtype=torch.uint8, device="cuda")
        vc = torch.zeros_like(kc)
        ks = torch.zeros((B, L, Hkv), dtype=torch.float32, device="cuda")
        vs = torch.zeros_like(ks)
        q_out = torch.empty_like(q)
        pos = torch.from_numpy(inp.positions).cuda()
        call = replayed(lambda: da.gqa_append_rope_fp8(q, kn, vn, pos, kc, vc, ks, vs, q_out=q_out))
        # bytes: q read and written (bf16), k and v rows read (bf16) and written
        # (codes + one fp32 scale per row), positions
        alg = dict(cache=2 * B * Hkv * (D * 2 + D + 4), q=2 * B * Hq * D * 2, out=0,
                   flops=6 * B * (Hq + Hkv) * (D // 2))
        alg["total"] = alg["cache"] + alg["q"] + 4 * B
        info = dict(batch=B, q_heads=Hq, kv_heads=Hkv, head_dim=D, max_seq_len=L, rotary_dim=D,
                    cache="e4m3, scale per (token, KV head) computed", rope="half pairs, base 10000")
        return [[("gqa_append_rope_fp8", call)]], alg, info, inp
    B, H, L = 64, 128, 4096
    inp = W.make_mla_append(B, H, L, cfg=3)
    qr, kvn = to_dev_bf16(inp.q), to_dev_bf16(inp.k_new)
    cache = torch.zeros((B, L, 576), dtype=torch.bfloat16, device="cuda")
    q_out = torch.empty_like(qr)
    pos = torch.from_numpy(inp.positions).cuda()

    call = replayed(lambda: da.mla_append_rope(qr, kvn, pos, cache, q_rope_out=q_out))
    alg = dict(cache=2 * B * 576 * 2, q=2 * B * H * 64 * 2, out=0, flops=6 * B * (H + 1) * 32)
    alg["total"] = alg["cache"] + alg["q"] + 4 * B
    info = dict(batch=B, heads=H, row=576, max_seq_len=L, rotary_dim=64, rope="half pairs, base 10000")
    return [[("mla_append_rope", call)]], alg, info, inp


def setup_gqa_fp8_paged(cfg, layout="head"):
    """The fp8 workload of `cfg` over paged pools: codes and per-(token, KV
    head) scales in 32-row pages placed in a seeded random physical order.
    layout "head": each page's codes stored [Hkv, 32, D]; "token": [32, Hkv,
    D]. Scales [pages, 32, Hkv] in both."""
    import torch
    import workloads as W
    import decode_attention_kv_bf16_amd as da
    inp = W.make_gqa_fp8_config(cfg)
    lens = inp.seq_lens
    ps = 32
    table, n_pages = W.make_block_table(lens, ps, seed=cfg, spare_pages=0)
    pools = [W.paginate(x, lens, table, n_pages, ps, 0) for x in (inp.k, inp.v, inp.k_scale, inp.v_scale)]
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    first = [head_major_codes(x) if layout == "head" else d(x) for x in pools[:2]] + [d(x) for x in pools[2:]]
    fp = sum(t.numel() * t.element_size() for t in first)
    n_copies = max(1, math.ceil(MALL_GUARD_BYTES / fp))
    copies = [first] + [[clone_view(t) if t.dim() == 4 else t.clone() for t in first] for _ in range(n_copies - 1)]
    tab = d(table)
    q = to_dev_bf16(inp.q)
    sl = torch.from_numpy(lens).cuda()
    B, Hq, D = q.shape
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    calls = []
    for kp, vp, ksp, vsp in copies:
        def call(kp=kp, vp=vp, ksp=ksp, vsp=vsp):
            da.gqa_decode_fp8_paged(q, kp, vp, ksp, vsp, tab, ps, sl, max_seq_len=inp.k.shape[1],
                                    softmax_scale=inp.scale, out=out, lse=lse)
        calls.append([("gqa_decode_fp8_paged", call)])
    alg = gqa_alg(B, Hq, inp.k.shape[2], D, int(lens.sum()), elem=1)
    scale_bytes = 2 * int(lens.sum()) * inp.k.shape[2] * 4
    table_bytes = table.size * 4
    alg["cache"] += scale_bytes + table_bytes
    alg["total"] += scale_bytes + table_bytes
    info = dict(batch=B, q_heads=Hq, kv_heads=int(inp.k.shape[2]), head_dim=D, seq_len=int(lens.max()),
                page_size=ps, cache="e4m3 + fp32 scale per (token, KV head), paged",
                codes="head-major pages [pages, Hkv, 32, D]" if layout == "head" else
                "token-major pages [pages, 32, Hkv, D]",
                cache_copies=len(copies))
    return calls, alg, info, (inp, dict(pools=pools, table=table))


def measured_traffic(workload, name):
    """HBM bytes per launch of kernel `name` in bench workload `workload`
    (its --workload value) from the committed rocprofv3 counter runs
    (profiles/hbm_traffic.json), if they were taken on the current kernel
    source; otherwise None."""
    from decode_attention_kv_bf16_amd.profiling import source_sha256
    path = os.path.join(PROFILE_DIR, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload, {}).get(name)
    if not rec or rec.get("source_sha256") != source_sha256(name):
        return None
    return round(rec["bytes_per_launch"])


def run_gpu(args):
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    import decode_attention_kv_bf16_amd as da
    da.lib()
    plans = []
    if args.workload in ("step", "gqa"):
        plans.append(("gqa", setup_gqa(2)))
    if args.workload in ("step", "mla"):
        plans.append(("mla", setup_mla(3)))
    if args.workload == "mla-long":
        plans.append(("mla", setup_mla(4)))
    if args.workload == "gqa-ragged":
        plans.append(("gqa", setup_gqa(5)))
    if args.workload == "gqa-paged":
        plans.append(("gqa-paged", setup_gqa_paged(2)))
    if args.workload == "mla-paged":
        plans.append(("mla-paged", setup_mla_paged(3)))
    if args.workload == "gqa-fp8":
        plans.append(("gqa-fp8", setup_gqa_fp8(2)))
    if args.workload == "gqa-fp8-token-major":
        plans.append(("gqa-fp8", setup_gqa_fp8(2, "token")))
    if args.workload == "gqa-fp8-paged":
        plans.append(("gqa-fp8-paged", setup_gqa_fp8_paged(2)))
    if args.workload == "gqa-fp8-paged-token-major":
        plans.append(("gqa-fp8-paged", setup_gqa_fp8_paged(2, "token")))
    if args.workload == "mla-fp8":
        plans.append(("mla-fp8", setup_mla_fp8(3)))
    if args.workload == "mla-fp8-paged":
        plans.append(("mla-fp8-paged", setup_mla_fp8_paged(3)))
    if args.workload == "gqa-window":
        plans.append(("gqa-window", setup_gqa_window()))
    if args.workload == "append":
        plans.append(("gqa-append", setup_append("gqa-append")))
        plans.append(("mla-append", setup_append("mla-append")))
    if args.workload == "append-fp8":
        plans.append(("gqa-append-fp8", setup_append("gqa-append-fp8")))
    n_rot = max(len(p[1][0]) for p in plans)

    def step_calls(i):
        seq = []
        for _, (calls, _, _, _) in plans:
            seq.extend(calls[i % len(calls)])
        return seq

    names = [n for n, _ in step_calls(0)]
    log(f"kernels per step: {names}; rotating {n_rot} input copies")
    for i in range(args.warmup):
        for _, fn in step_calls(i):
            fn()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    hev = HipTimingEvents()

    # Probe pass (untimed, after the warm-up): an event between every two
    # launches gives the per-kernel breakdown and picks the dominant kernel.
    n_probe = max(3, min(args.steps, 10))
    ev = [[hev.create() for _ in range(len(names) + 1)] for _ in range(n_probe)]
    for i in range(n_probe):
        e = ev[i]
        hev.record(e[0], stream)
        for j, (_, fn) in enumerate(step_calls(args.warmup + i)):
            fn()
            hev.record(e[j + 1], stream)
    torch.cuda.synchronize()
    per_kernel = {n: float(np.mean([hev.elapsed_ms(ev[i][j], ev[i][j + 1]) for i in range(n_probe)]))
                  for j, n in enumerate(names)}
    dom = max(per_kernel, key=per_kernel.get)
    dom_idx = names.index(dom)

    # Timed region: exactly K steps, synchronised on both sides, with nothing
    # between the launches (an event between two kernels makes the second wait
    # for the first to finish completely, so consecutive kernels no longer
    # overlap at their edges: the step would be measured slower than it runs).
    step_ev = (hev.create(), hev.create())
    base = args.warmup + n_probe
    torch.cuda.synchronize()
    with Telemetry() as tele:
        t0 = time.perf_counter()
        hev.record(step_ev[0], stream)
        for i in range(args.steps):
            for _, fn in step_calls(base + i):
                fn()
        hev.record(step_ev[1], stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    ev_step_ms = hev.elapsed_ms(*step_ev) / args.steps

    # Step distribution: K more steps with an event at every step boundary
    # (none between the kernels of a step): median, p10 and p90 per step.
    base += args.steps
    bound_ev = [hev.create() for _ in range(args.steps + 1)]
    hev.record(bound_ev[0], stream)
    for i in range(args.steps):
        for _, fn in step_calls(base + i):
            fn()
        hev.record(bound_ev[i + 1], stream)
    torch.cuda.synchronize()
    per_step = np.array([hev.elapsed_ms(bound_ev[i], bound_ev[i + 1]) for i in range(args.steps)])
    step_stats = dict(median=round(float(np.median(per_step)), 4), p10=round(float(np.percentile(per_step, 10)), 4),
                      p90=round(float(np.percentile(per_step, 90)), 4))

    # Roofline pass: K more steps in which events on the launch stream bracket
    # every launch of the dominant kernel; its average duration.
    # When a step takes the GPU less time than Python needs to issue it (the
    # few-microsecond append kernels), an event pair would time the issue gap,
    # not the kernel. Then the pass starts behind a GPU busy-wait (a spin
    # kernel of known length) long enough for every launch and event of the
    # pass to be queued first, so the kernels run back to back as in a loop
    # that is not limited by its host.
    dom_ev = [(hev.create(), hev.create()) for _ in range(args.steps)]
    base += args.steps
    probe_step_ms = sum(per_kernel.values())
    if probe_step_ms < 0.03:
        cal = (hev.create(), hev.create())
        hev.record(cal[0], stream)
        torch.cuda._sleep(1_000_000)
        hev.record(cal[1], stream)
        torch.cuda.synchronize()
        ms_per_mcycle = max(hev.elapsed_ms(*cal), 1e-3)
        wanted_ms = 0.05 * args.steps * len(names) + 5.0     # generous: 50 us of issue per launch
        torch.cuda._sleep(int(wanted_ms / ms_per_mcycle * 1_000_000))
        roofline_queued = True
    else:
        roofline_queued = False
    for i in range(args.steps):
        for j, (_, fn) in enumerate(step_calls(base + i)):
            if j == dom_idx:
                hev.record(dom_ev[i][0], stream)
                fn()
                hev.record(dom_ev[i][1], stream)
            else:
                fn()
    torch.cuda.synchronize()
    dom_ms = float(np.mean([hev.elapsed_ms(a, b) for a, b in dom_ev]))
    hev.close()

    total_bytes = sum(p[1][1]["total"] for p in plans)
    total_flops = sum(p[1][1]["flops"] for p in plans)
    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    tflops = total_flops / (ms_per_step * 1e-3) / 1e12

    # dominant kernel's roofline
    kind, (calls, alg, info, _) = next(p for p in plans
                                       if any(dom == n for n, _ in p[1][0][0]))
    if dom in ("gqa_split_pass", "gqa_window"):
        dom_bytes = alg["cache"] + alg["q"]
    elif dom == "gqa_decode_fp8_paged":
        dom_bytes = alg["cache"] + alg["q"]
    elif dom in ("mla_attend", "mla_attend_paged"):
        dom_bytes = alg["cache"]
    else:
        dom_bytes = alg["total"]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(args.workload, dom),
                "alg_bytes_per_launch": int(dom_bytes), "avg_launch_us": round(dom_ms * 1e3, 2),
                "launches_queued_behind_spin": roofline_queued}

    paths = {}
    for kind, (calls, alg, info, _) in plans:
        ks = [n for n, _ in calls[0]]
        t_ms = sum(per_kernel[n] for n in ks)
        entry = dict(info)
        entry.update(probe_kernels_us={n: round(per_kernel[n] * 1e3, 2) for n in ks},
                     time_us=round(t_ms * 1e3, 2), alg_bytes=int(alg["total"]),
                     alg_gbs=round(alg["total"] / (t_ms * 1e-3) / 1e9, 1),
                     cache_gbs=round(alg["cache"] / (t_ms * 1e-3) / 1e9, 1),
                     tflops=round(alg["flops"] / (t_ms * 1e-3) / 1e12, 2),
                     hbm_frac=round(alg["total"] / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
        if kind.startswith("mla"):
            entry["mfma_frac"] = round(alg["flops"] / (t_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        entry["binding_roofline"] = binding_roofline(alg, t_ms)
        paths[kind] = entry

    if args.workload == "step" and args.extra_paths:
        # timed on their own after the headline step (not part of it):
        # long-context MLA, ragged MHA, then E4M3 caches of the step's GQA and
        # MLA shapes
        for key, setup in (("mla_long", lambda: setup_mla(4)), ("gqa_ragged", lambda: setup_gqa(5)),
                           ("gqa_fp8", lambda: setup_gqa_fp8(2)),
                           ("gqa_fp8_token_major", lambda: setup_gqa_fp8(2, "token")),
                           ("mla_fp8", lambda: setup_mla_fp8(3))):
            paths[key] = time_path(key, setup(), args, hev, stream)
            torch.cuda.empty_cache()
    ceiling = hbm_ceiling(hev, stream) if args.hbm_probe else None

    prop = torch.cuda.get_device_properties(0)
    res = dict(metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms_per_step, 4), higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
               config=dict(workload=workload_name(args.workload), parallelism="single-gpu"),
               tflops=round(tflops, 2), event_ms_per_step=round(ev_step_ms, 4), step_ms=step_stats,
               roofline=roofline, paths=paths,
               device=dict(name=prop.name, cus=prop.multi_processor_count,
                           arch=getattr(prop, "gcnArchName", ""), rocm=rocm_version(),
                           timed_region=tele.summary(), measured_hbm=ceiling))
    return res, plans


def hbm_ceiling(hev, stream, read_mib=2048, copy_mib=1024, reps=8):
    """The device's measured streaming rates, context for the roofline
    fractions: the library's read probe over a read_mib buffer and its copy
    probe over copy_mib (read + write bytes counted), over a few grid sizes
    (workgroups per CU) and load depths, median of `reps` event-timed launches
    each. The best shape is the ceiling; every shape is reported."""
    import torch
    import decode_attention_kv_bf16_amd as da
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"read_bytes": read_mib << 20, "copy_bytes": copy_mib << 20, "per_shape": {}}
    buf = torch.empty(read_mib << 20, dtype=torch.uint8, device="cuda")
    buf.random_(0, 256)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ev = [hev.create() for _ in range(2 * reps)]

    def median_ms(launch):
        for _ in range(2):
            launch()
        for r in range(reps):
            hev.record(ev[2 * r], stream)
            launch()
            hev.record(ev[2 * r + 1], stream)
        stream.synchronize()
        return float(np.median([hev.elapsed_ms(ev[2 * r], ev[2 * r + 1]) for r in range(reps)]))

    best = {"read": (0.0, None), "copy": (0.0, None)}
    for wg_per_cu, depth in ((1, 4), (1, 8), (1, 16), (1.5, 4), (1.5, 8), (2, 4), (2, 8)):
        blocks = int(wg_per_cu * cus)
        tbs = buf.numel() / median_ms(lambda: da.probe_stream_read(buf, sink, blocks, depth)) / 1e9
        key = f"read_{wg_per_cu}wg_per_cu_depth{depth}"
        out["per_shape"][key] = round(tbs, 3)
        best["read"] = max(best["read"], (tbs, key))
    del buf
    src = torch.empty(copy_mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for wg_per_cu, depth in ((1, 4), (1, 8), (2, 4), (2, 8)):
        blocks = int(wg_per_cu * cus)
        tbs = 2 * src.numel() / median_ms(lambda: da.probe_stream_copy(src, dst, blocks, depth)) / 1e9
        key = f"copy_{wg_per_cu}wg_per_cu_depth{depth}"
        out["per_shape"][key] = round(tbs, 3)
        best["copy"] = max(best["copy"], (tbs, key))
    del src, dst
    torch.cuda.empty_cache()
    out["read_tb_s"], out["read_shape"] = round(best["read"][0], 3), best["read"][1]
    out["copy_tb_s"], out["copy_shape"] = round(best["copy"][0], 3), best["copy"][1]
    return out


def time_path(key, plan, args, hev, stream):
    """A workload timed alone: warm-up, then its calls back to back with an
    event at every call boundary (median, p10, p90 per call) and, in a second
    pass, events around its dominant kernel (the attention or split pass)."""
    import torch
    calls, alg, info, _ = plan
    names = [n for n, _ in calls[0]]
    n = len(calls)
    for i in range(max(args.warmup, 20)):
        for _, fn in calls[i % n]:
            fn()
    steps = max(args.steps, 20)
    ev = [hev.create() for _ in range(steps + 1)]
    torch.cuda.synchronize()
    with Telemetry() as tele:
        hev.record(ev[0], stream)
        for i in range(steps):
            for _, fn in calls[i % n]:
                fn()
            hev.record(ev[i + 1], stream)
        torch.cuda.synchronize()
    t = np.array([hev.elapsed_ms(ev[i], ev[i + 1]) for i in range(steps)])
    # the attention kernel (or the whole call, for one-call paths)
    dom = "mla_attend" if "mla_attend" in names else "gqa_split_pass" if "gqa_split_pass" in names else names[0]
    j = names.index(dom)
    dev = [(hev.create(), hev.create()) for _ in range(steps)]
    for i in range(steps):
        for k, (_, fn) in enumerate(calls[i % n]):
            if k == j:
                hev.record(dev[i][0], stream)
                fn()
                hev.record(dev[i][1], stream)
            else:
                fn()
    torch.cuda.synchronize()
    dom_ms = float(np.mean([hev.elapsed_ms(a, b) for a, b in dev]))
    med = float(np.median(t))
    dom_bytes = (alg["cache"] if dom == "mla_attend" else alg["cache"] + alg["q"] if dom == "gqa_split_pass"
                 else alg["total"])
    entry = dict(info)
    entry.update(time_us=round(med * 1e3, 2), p10_us=round(float(np.percentile(t, 10)) * 1e3, 2),
                 p90_us=round(float(np.percentile(t, 90)) * 1e3, 2), alg_bytes=int(alg["total"]),
                 alg_gbs=round(alg["total"] / (med * 1e-3) / 1e9, 1),
                 tflops=round(alg["flops"] / (med * 1e-3) / 1e12, 2),
                 roofline_frac=round(alg["total"] / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 dominant_kernel=dict(kernel=dom, avg_launch_us=round(dom_ms * 1e3, 2),
                                      hbm_frac=round(dom_bytes / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)),
                 binding_roofline=binding_roofline(alg, med),
                 timed_region=tele.summary())
    return entry


def workload_name(w):
    return {"step": "llama3-8b-gqa-b32-l4096 + deepseek-v3-mla-b64-l4096",
            "gqa": "llama3-8b-gqa-b32-l4096", "mla": "deepseek-v3-mla-b64-l4096",
            "mla-long": "deepseek-v3-mla-longctx-b4-l16k-32k",
            "gqa-ragged": "llama2-7b-mha-ragged-b64-l1-8192",
            "gqa-paged": "llama3-8b-gqa-b32-l4096-paged16",
            "mla-paged": "deepseek-v3-mla-b64-l4096-paged16",
            "gqa-fp8": "llama3-8b-gqa-b32-l4096-fp8e4m3-headmajor",
            "gqa-fp8-token-major": "llama3-8b-gqa-b32-l4096-fp8e4m3-tokenmajor",
            "gqa-window": "mistral-7b-shape-gqa-b32-l8192-window4096",
            "gqa-fp8-paged": "llama3-8b-gqa-b32-l4096-fp8e4m3-paged32-headmajor",
            "gqa-fp8-paged-token-major": "llama3-8b-gqa-b32-l4096-fp8e4m3-paged32-tokenmajor",
            "mla-fp8": "deepseek-v3-mla-b64-l4096-fp8e4m3-nope-rope-scales",
            "mla-fp8-paged": "deepseek-v3-mla-b64-l4096-fp8e4m3-nope-rope-scales-paged16",
            "append-fp8": "cache append + rope into e4m3: llama3-8b-gqa-b32-l4096",
            "append": "cache append + rope: llama3-8b-gqa-b32-l4096 + deepseek-v3-mla-b64-l4096"}[w]


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the same workload
# ----------------------------------------------------------------------------

def oracle_calls(kind, inp):
    """One closure per sequence that runs the fp64 oracle on that sequence
    alone, with the cached rows it covers (1 per sequence for appends).
    Inputs are widened to fp64 outside the closures (not timed)."""
    from oracle.attention import (gqa_decode_paged_ref, gqa_decode_ref, mla_absorbed_paged_ref,
                                  mla_absorbed_ref)
    from oracle.fp8 import (gqa_append_rope_fp8_ref, gqa_decode_fp8_paged_ref, gqa_decode_fp8_ref,
                            mla_absorbed_fp8_paged_ref, mla_absorbed_fp8_ref)
    from oracle.rope import gqa_append_rope_ref, mla_append_rope_ref
    import workloads as W
    f = (lambda a: W.bf16_to_f32(a).astype(np.float64))
    pools = None
    if kind.endswith("-paged"):
        inp, pools = inp
    calls = []
    if "-append" in kind:
        for b in range(len(inp.positions)):
            if kind == "gqa-append-fp8":
                args = (inp.f64("q")[b:b + 1], inp.f64("k_new")[b:b + 1], inp.f64("v_new")[b:b + 1],
                        inp.positions[b:b + 1], 4096, inp.q.shape[2], 0)
                calls.append((lambda a=args: gqa_append_rope_fp8_ref(*a), 1))
                continue
            # one sequence per call into a one-page pool (page size 16): the
            # same rotation and row write, without copying a whole cache
            tab = np.zeros((1, -(-4096 // 16)), np.int32)
            if kind == "gqa-append":
                Hkv, D = inp.k_new.shape[1], inp.k_new.shape[2]
                pool = np.zeros((1, 16, Hkv, D))
                args = (inp.f64("q")[b:b + 1], inp.f64("k_new")[b:b + 1], inp.f64("v_new")[b:b + 1],
                        inp.positions[b:b + 1], pool, pool, 4096, D, 0)
                calls.append((lambda a=args, t=tab: gqa_append_rope_ref(*a, block_table=t, page_size=16), 1))
            else:
                pool = np.zeros((1, 16, 576))
                args = (inp.f64("q")[b:b + 1], inp.f64("k_new")[b:b + 1], inp.positions[b:b + 1],
                        pool, 4096, 64, 0)
                calls.append((lambda a=args, t=tab: mla_append_rope_ref(*a, block_table=t, page_size=16), 1))
        return calls
    lens = inp.seq_lens
    for b in range(len(lens)):
        L = int(lens[b])
        sl = lens[b:b + 1]
        if kind in ("gqa-paged", "mla-paged", "gqa-fp8-paged", "mla-fp8-paged"):
            ps = 32 if kind == "gqa-fp8-paged" else PAGE_SIZE
            pages = pools["table"][b, :max(1, -(-L // ps))]
            # only the sequence's own pages, renumbered, go to the oracle
            tab = np.arange(len(pages), dtype=np.int32)[None]
        if kind == "gqa-paged":
            args = (f(inp.q[b:b + 1]), f(pools["k_pool"][pages]), f(pools["v_pool"][pages]), tab,
                    PAGE_SIZE, sl, inp.scale)
            calls.append((lambda a=args: gqa_decode_paged_ref(*a), L))
        elif kind == "mla-paged":
            args = (f(inp.q_nope[b:b + 1]), f(inp.q_rope[b:b + 1]), f(pools["pool"][pages]), tab,
                    PAGE_SIZE, sl, f(inp.w_uk), f(inp.w_uv), inp.scale)
            calls.append((lambda a=args: mla_absorbed_paged_ref(*a), L))
        elif kind == "gqa-fp8-paged":
            kp, vp, ksp, vsp = pools["pools"]
            args = (f(inp.q[b:b + 1]), kp[pages], vp[pages], ksp[pages], vsp[pages], tab, 32, sl, inp.scale)
            calls.append((lambda a=args: gqa_decode_fp8_paged_ref(*a), L))
        elif kind == "gqa-fp8":
            args = (f(inp.q[b:b + 1]), inp.k[b:b + 1, :L], inp.v[b:b + 1, :L], inp.k_scale[b:b + 1, :L],
                    inp.v_scale[b:b + 1, :L], sl, inp.scale)
            calls.append((lambda a=args: gqa_decode_fp8_ref(*a), L))
        elif kind == "mla-fp8-paged":
            cp, snp, srp = pools["pools"]
            args = (f(inp.q_nope[b:b + 1]), f(inp.q_rope[b:b + 1]), cp[pages], snp[pages], srp[pages], tab,
                    PAGE_SIZE, sl, f(inp.w_uk), f(inp.w_uv), inp.scale)
            calls.append((lambda a=args: mla_absorbed_fp8_paged_ref(*a), L))
        elif kind == "mla-fp8":
            args = (f(inp.q_nope[b:b + 1]), f(inp.q_rope[b:b + 1]), inp.cache[b:b + 1, :L],
                    inp.scale_nope[b:b + 1, :L], inp.scale_rope[b:b + 1, :L], sl, f(inp.w_uk), f(inp.w_uv),
                    inp.scale)
            calls.append((lambda a=args: mla_absorbed_fp8_ref(*a), L))
        elif kind in ("gqa", "gqa-window"):
            conv = f if inp.dtype == "bf16" else (lambda a: a.astype(np.float64))
            args = (conv(inp.q[b:b + 1]), conv(inp.k[b:b + 1, :L]), conv(inp.v[b:b + 1, :L]), sl, inp.scale)
            w = WINDOW if kind == "gqa-window" else 0
            calls.append((lambda a=args, w=w: gqa_decode_ref(*a, window=w), min(L, w) if w else L))
        else:
            args = (f(inp.q_nope[b:b + 1]), f(inp.q_rope[b:b + 1]), f(inp.cache[b:b + 1, :L]), sl,
                    f(inp.w_uk), f(inp.w_uv), inp.scale)
            calls.append((lambda a=args: mla_absorbed_ref(*a), L))
    return calls


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(plans, budget_s):
    """The fp64 oracle on the host cores, timed for one step's worth of work.

    For every path of the step the oracle runs one sequence per call. The
    sample is every sequence when that fits the time budget, else the first
    sequences of each path; the time of the whole step is the sample's time
    scaled by (the path's cached rows / the sample's rows). Each timing is the
    median of 3 runs, with numpy's BLAS at all host threads and again at one
    thread. value = the step's algorithmic bytes (weights counted once per
    call, as for the GPU) / the all-thread step time, in GB/s. `seconds` is
    that scaled step time; `wall_seconds` the host time the whole measurement
    took."""
    t_start = time.perf_counter()
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = 1
    paths = []
    for kind, (calls, alg, info, inp) in plans:
        oc = oracle_calls(kind, inp)
        paths.append(dict(kind=kind, calls=oc, rows=sum(r for _, r in oc), alg_bytes=int(alg["total"])))
    # pilot: each path's first call, to size the sample
    for p in paths:
        t = time.perf_counter()
        p["calls"][0][0]()
        p["pilot"] = max(time.perf_counter() - t, 1e-6)
    # 3 runs at all threads and 3 at one thread, one thread assumed up to 4x
    # slower: one all-thread run may take budget / 15
    per_path = budget_s / 15.0 / len(paths)
    for p in paths:
        n = int(max(1, min(len(p["calls"]), per_path // p["pilot"])))
        p["sample"] = p["calls"][:n]
        p["sample_rows"] = max(1, sum(r for _, r in p["sample"]))

    def step_seconds():
        total = 0.0
        for p in paths:
            t = time.perf_counter()
            for fn, _ in p["sample"]:
                fn()
            total += (time.perf_counter() - t) * p["rows"] / p["sample_rows"]
        return total

    all_t = float(np.median([step_seconds() for _ in range(3)]))
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            one_t = float(np.median([step_seconds() for _ in range(3)]))
    else:  # pragma: no cover
        one_t = all_t
    step_bytes = sum(p["alg_bytes"] for p in paths)
    sample = "; ".join(f"{p['kind']}: {len(p['sample'])} of {len(p['calls'])} sequences" for p in paths)
    return dict(value=round(step_bytes / all_t / 1e9, 4), unit="GB/s", cores=int(threads), kind="oracle",
                sample=sample + ", step time scaled by cached rows, median of 3 runs",
                seconds=all_t, step_alg_bytes=int(step_bytes),
                wall_seconds=round(time.perf_counter() - t_start, 2),
                single_thread=dict(value=round(step_bytes / one_t / 1e9, 4), seconds=round(one_t, 4)),
                host_cpus=os.cpu_count(), cpu_model=cpu_model())


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="step",
                    choices=["step", "gqa", "mla", "mla-long", "gqa-ragged", "gqa-paged",
                             "mla-paged", "gqa-fp8", "append", "gqa-window",
                             "append-fp8", "gqa-fp8-paged", "mla-fp8", "mla-fp8-paged",
                             "gqa-fp8-token-major", "gqa-fp8-paged-token-major"])
    ap.add_argument("--cpu-budget", type=float, default=40.0,
                    help="seconds of oracle time for the CPU baseline (0 disables)")
    ap.add_argument("--no-extra-paths", dest="extra_paths", action="store_false",
                    help="skip timing the long-context MLA and ragged MHA workloads after the step")
    ap.add_argument("--no-hbm-probe", dest="hbm_probe", action="store_false",
                    help="skip measuring the device's streaming read and copy rates")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB after the timed "
                         "steps (a kernel of known traffic, to scale hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path).", file=sys.stderr)
        raise SystemExit(2)
    res, plans = run_gpu(args)
    if args.calibration_copy_mib > 0:
        import torch
        n = args.calibration_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["calibration_copy_bytes"] = n
    if args.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(plans, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
