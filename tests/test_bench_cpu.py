"""Host logic of bench.py: the one-GPU contract, workload names and the CPU
baseline leg (the fp64 oracle on a bounded sample), on tiny inputs."""
import os
import subprocess
import sys

import numpy as np

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_every_workload_has_a_name():
    for w in ("step", "gqa", "mla", "mla-long", "gqa-ragged", "gqa-paged", "mla-paged", "gqa-fp8",
              "append", "gqa-window", "append-fp8", "gqa-fp8-paged"):
        assert bench.workload_name(w)


def test_paged_pools_hold_every_row_once():
    inp = W.make_gqa(3, 4, 2, 64, [40, 16, 1], "bf16", seed=2, max_seq_len=48)
    (kp,), table = bench.paged_pools(inp.seq_lens, [inp.k], seed=1)
    assert kp.shape[1] == bench.PAGE_SIZE and kp.shape[0] == 3 + 1 + 1
    for b, L in enumerate(inp.seq_lens):
        for t in range(L):
            page = table[b, t // bench.PAGE_SIZE]
            assert np.array_equal(kp[page, t % bench.PAGE_SIZE], inp.k[b, t])


def test_cpu_baseline_on_contiguous_and_paged_plans():
    g = W.make_gqa(2, 8, 2, 128, [64, 33], "bf16", seed=3, max_seq_len=64)
    m = W.make_mla(2, 16, [40, 7], seed=4, max_seq_len=48)
    (kp, vp), tg = bench.paged_pools(g.seq_lens, [g.k, g.v], seed=5)
    (pool,), tm = bench.paged_pools(m.seq_lens, [m.cache], seed=6)
    f8 = W.make_gqa_fp8(2, 8, 2, 128, [40, 9], seed=7)
    plans = [("gqa", (None, None, None, g)), ("mla", (None, None, None, m)),
             ("gqa-fp8", (None, None, None, f8)),
             ("gqa-paged", (None, None, None, (g, dict(k_pool=kp, v_pool=vp, table=tg)))),
             ("mla-paged", (None, None, None, (m, dict(pool=pool, table=tm)))),
             ("gqa-append", (None, dict(total=2000), None, W.make_gqa_append(2, 8, 2, 128, 4096))),
             ("mla-append", (None, dict(total=2000), None, W.make_mla_append(2, 16, 4096))),
             ("gqa-append-fp8", (None, dict(total=2000), None, W.make_gqa_append(2, 8, 2, 128, 4096)))]
    res = bench.cpu_baseline(plans, budget_s=4.0)
    assert res["kind"] == "oracle" and res["value"] > 0 and res["cores"] >= 1
    for kind in ("gqa", "mla", "gqa-paged", "mla-paged", "gqa-fp8", "gqa-append", "mla-append",
                 "gqa-append-fp8"):
        assert f"{kind}: 2 of 2 sequences" in res["sample"]
