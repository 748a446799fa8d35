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
              "append", "gqa-window", "append-fp8", "gqa-fp8-paged", "mla-fp8", "mla-fp8-paged",
              "gqa-fp8-token-major", "gqa-fp8-paged-token-major"):
        assert bench.workload_name(w)


def test_head_major_codes_view_the_same_values():
    # the head-major storage, seen through the strided view, holds every code
    # where the token-major array has it (CPU tensors here; the bench puts
    # them on the GPU)
    import torch
    x = np.random.default_rng(3).integers(0, 255, (2, 5, 3, 4), dtype=np.uint8)
    base = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3)))
    view = base.permute(0, 2, 1, 3)
    assert view.shape == x.shape and view.stride() == (3 * 5 * 4, 4, 5 * 4, 1)
    assert np.array_equal(view.numpy(), x)
    c = bench.clone_view(view)
    assert c.stride() == view.stride() and torch.equal(c, view) and c.data_ptr() != view.data_ptr()


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
    m8 = W.make_mla_fp8(2, 16, [33, 5], seed=8, max_seq_len=40)
    ga = bench.gqa_alg(2, 8, 2, 128, int(g.seq_lens.sum()))
    ma = bench.mla_alg(2, 16, int(m.seq_lens.sum()))
    fa = bench.gqa_alg(2, 8, 2, 128, int(f8.seq_lens.sum()), elem=1)
    m8a = bench.mla_alg(2, 16, int(m8.seq_lens.sum()), elem=1)
    (cp, snp, srp), t8 = bench.paged_pools(m8.seq_lens, [m8.cache, m8.scale_nope, m8.scale_rope], seed=9)
    plans = [("gqa", (None, ga, None, g)), ("mla", (None, ma, None, m)),
             ("gqa-fp8", (None, fa, None, f8)), ("mla-fp8", (None, m8a, None, m8)),
             ("mla-fp8-paged", (None, m8a, None, (m8, dict(pools=(cp, snp, srp), table=t8)))),
             ("gqa-paged", (None, ga, None, (g, dict(k_pool=kp, v_pool=vp, table=tg)))),
             ("mla-paged", (None, ma, None, (m, dict(pool=pool, table=tm)))),
             ("gqa-append", (None, dict(total=2000), None, W.make_gqa_append(2, 8, 2, 128, 4096))),
             ("mla-append", (None, dict(total=2000), None, W.make_mla_append(2, 16, 4096))),
             ("gqa-append-fp8", (None, dict(total=2000), None, W.make_gqa_append(2, 8, 2, 128, 4096)))]
    res = bench.cpu_baseline(plans, budget_s=30.0)   # room for every sequence even on a loaded host
    assert res["kind"] == "oracle" and res["value"] > 0 and res["cores"] >= 1
    for kind in ("gqa", "mla", "gqa-paged", "mla-paged", "gqa-fp8", "mla-fp8", "mla-fp8-paged", "gqa-append",
                 "mla-append", "gqa-append-fp8"):
        assert f"{kind}: 2 of 2 sequences" in res["sample"]
    # one byte basis with the GPU figure: the step's algorithmic bytes (MLA
    # weights once per call, not once per sequence) over the oracle's seconds
    step_bytes = 2 * ga["total"] + 2 * ma["total"] + fa["total"] + 2 * m8a["total"] + 3 * 2000
    assert res["step_alg_bytes"] == step_bytes
    assert abs(res["value"] - step_bytes / res["seconds"] / 1e9) <= 1e-4 * res["value"] + 1e-4
    assert res["single_thread"]["seconds"] > 0 and res["cpu_model"]


def test_cpu_baseline_scales_a_partial_sample_by_rows():
    # a budget too small for every sequence: the first sequences are timed
    # and the step time is scaled by the path's rows over the sample's
    g = W.make_gqa(6, 8, 2, 128, [64, 32, 32, 32, 32, 32], "bf16", seed=3, max_seq_len=64)
    ga = bench.gqa_alg(6, 8, 2, 128, int(g.seq_lens.sum()))
    res = bench.cpu_baseline([("gqa", (None, ga, None, g))], budget_s=1e-9)
    assert "gqa: 1 of 6 sequences" in res["sample"]
    assert abs(res["value"] - ga["total"] / res["seconds"] / 1e9) <= 1e-4 * res["value"] + 1e-4


def test_binding_roofline_picks_the_longer_bound():
    # DeepSeek-V3 MLA (B 64, L 4096) in bf16 is HBM-bound on spec numbers; in E4M3 (half the
    # cache bytes, the same matrix work) the matrix cores bind
    bf = bench.mla_alg(64, 128, 64 * 4096)
    f8 = bench.mla_alg(64, 128, 64 * 4096, elem=1)
    assert bench.binding_roofline(bf, 1.0)["bound"] == "hbm"
    assert bench.binding_roofline(f8, 1.0)["bound"] == "mfma"
    r = bench.binding_roofline(f8, 0.060)
    assert abs(r["frac"] - f8["flops"] / 2.5e15 / 0.060e-3) < 1e-3


def test_profile_summaries_name_every_attention_kernel():
    from decode_attention_kv_bf16_amd.profiling import short_name, source_sha256
    ns = "void da::(anonymous namespace)::"
    assert short_name(ns + "mla_attend32_kernel<4, false>(da::MlaArgs)") == "mla_attend"
    assert short_name(ns + "mla_attend32_kernel<4, true>(da::MlaArgs)") == "mla_attend_paged"
    assert short_name(ns + "mla_attend_kernel<1, 1, false>(da::MlaArgs)") == "mla_attend"
    assert short_name(ns + "mla_attend_fp8_kernel<4, false>(da::MlaArgs)") == "mla_attend_fp8"
    assert short_name(ns + "mla_attend_fp8_kernel<4, true>(da::MlaArgs)") == "mla_attend_fp8_paged"
    assert short_name("_ZN2da12_GLOBAL__N_119mla_attend32_kernelILi4ELb1EEEvNS_7MlaArgsE") == "mla_attend_paged"
    assert short_name(ns + "mla_merge_project_kernel(da::MlaArgs, int, int)") == "mla_merge_project"
    for k in ("mla_attend", "mla_attend_fp8", "mla_absorb", "gqa_split_pass"):
        assert len(source_sha256(k)) == 64
    assert short_name(ns + "stream_read_kernel<8>(unsigned int const*, long, unsigned int*)") == \
        "probe_stream_read"


def test_counter_summary_follows_the_derived_counter_definitions(tmp_path):
    """Two dispatches of one kernel, counters summed over 8 XCCs: the derived
    figures are rocprofv3's MfmaUtil, VALUBusy, LdsUtil and LdsBankConflict
    with GRBM_GUI_ACTIVE taken per XCC, and the clock is cycles / duration."""
    from decode_attention_kv_bf16_amd.profiling import counter_table
    hdr = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size",'
           '"Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count",'
           '"Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"')
    name = "void da::(anonymous namespace)::mla_attend32_kernel<4, false>(da::MlaArgs)"
    gui_per_xcc, dur_ns = 200_000, 100_000          # 2.0 GHz
    vals = {"GRBM_GUI_ACTIVE": 8 * gui_per_xcc,
            "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * gui_per_xcc * 1024,   # half of every SIMD's cycles
            "SQ_ACTIVE_INST_VALU": 0.25 * gui_per_xcc * 256,
            "SQ_LDS_IDX_ACTIVE": 0.2 * gui_per_xcc * 256,
            "SQ_LDS_BANK_CONFLICT": 0.04 * gui_per_xcc * 256}
    lines = [hdr]
    for disp in (1, 2):
        t0 = 1_000_000 * disp
        for c, v in vals.items():
            lines.append(f'{disp},{disp},"Agent 1",1,1,1,1,1,"{name}",256,0,0,8,0,32,"{c}",{v},{t0},{t0 + dur_ns}')
        lines.append(f'{disp + 9},{disp + 9},"Agent 1",1,1,1,1,1,"__amd_rocclr_copyBuffer",256,0,0,8,0,32,'
                     f'"GRBM_GUI_ACTIVE",5,{t0},{t0 + 10}')
    (tmp_path / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")
    rows = counter_table([str(tmp_path)])
    assert set(rows) == {"mla_attend"}
    r = rows["mla_attend"]
    assert r["dispatches"] == 2 and abs(r["duration_us"] - 100.0) < 1e-9
    assert abs(r["sclk_ghz"] - 2.0) < 1e-9
    assert abs(r["mfma_busy_pct"] - 50.0) < 1e-9
    assert abs(r["valu_busy_pct"] - 25.0) < 1e-9
    assert abs(r["lds_busy_pct"] - 20.0) < 1e-9
    assert abs(r["lds_conflicts_per_access"] - 0.04 / 0.16) < 1e-9


def test_parity_table_lists_every_check_and_the_mla_summary():
    from decode_attention_kv_bf16_amd.profiling import parity_table
    rec = {"exitstatus": 0, "checks": {
        "tests/test_gpu_mla.py::test_a :: mla config3": dict(max_row_rel_err=6e-3, max_lse_abs_err=2e-5,
                                                              out_rtol=1e-2, lse_atol=1e-3),
        "tests/test_gpu_gqa.py::test_b :: gqa config2": dict(max_row_rel_err=3e-3, max_lse_abs_err=1e-6,
                                                              out_rtol=1e-2, lse_atol=1e-3)}}
    text = parity_table(rec, "pytest tests -m gpu")
    assert "2 parity checks" in text and "MLA checks: 1" in text
    assert "| 6.00e-03 | 2.00e-05 |" in text and "| 3.00e-03 | 1.00e-06 |" in text
    assert "tests/" not in text.split("| test :: check |")[1]


def test_traffic_summary_scales_counters_by_the_copy_kernel(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by the factors
    that make the run's closing copy kernel read its known size, and the
    record lands under the bench workload and the kernel name."""
    import json
    from decode_attention_kv_bf16_amd import profiling
    monkeypatch.setattr(profiling, "PROFILE_DIR", str(tmp_path))
    hdr = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size",'
           '"Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count",'
           '"Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"')
    name = "void da::(anonymous namespace)::mla_attend32_kernel<4, false>(da::MlaArgs)"
    copy_bytes = 512 << 20

    def run_dir(counter, kernel_kib, copy_kib):
        d = tmp_path / counter
        d.mkdir()
        rows = [hdr]
        for disp, v in ((1, kernel_kib), (2, kernel_kib + 2.0)):
            rows.append(f'{disp},{disp},"Agent 1",1,1,1,1,1,"{name}",256,0,0,8,0,32,"{counter}",{v},0,10')
        rows.append(f'3,3,"Agent 1",1,1,1,1,1,"__amd_rocclr_copyBuffer",256,0,0,8,0,32,"{counter}",{copy_kib},0,10')
        (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
        return str(d)

    fetch = run_dir("FETCH_SIZE", 1000.0, copy_bytes / 1024 / 2)    # the copy's reads count half
    write = run_dir("WRITE_SIZE", 100.0, copy_bytes / 1024)
    profiling.main(["traffic", "--fetch", fetch, "--write", write, "--copy-bytes", str(copy_bytes),
                    "--fetch-command", "f", "--write-command", "w", "--workload", "mla test",
                    "--key", "mla", "--alg-bytes", '{"mla_attend": 2000000}',
                    "--out-md", str(tmp_path / "t.md")])
    rec = json.load(open(tmp_path / "hbm_traffic.json"))["mla"]["mla_attend"]
    assert abs(rec["fetch_factor"] - 2.0) < 1e-12 and abs(rec["write_factor"] - 1.0) < 1e-12
    assert abs(rec["bytes_per_launch"] - (1001.0 * 1024 * 2 + 101.0 * 1024)) < 1e-6
    assert rec["algorithmic_bytes"] == 2000000 and len(rec["source_sha256"]) == 64
