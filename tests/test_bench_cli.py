"""The benchmark's command-line contract on the host: it measures one GPU and refuses more,
with a message and a non-zero status, before touching any device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2
    assert "WORLD_SIZE 4" in r.stderr


def test_timing_events_find_the_loaded_hip_runtime():
    """The benchmark's timing events use the HIP runtime already mapped into the process (no
    library name is assumed) and read the fence-free event flag from the HIP headers."""
    sys.path.insert(0, ROOT)
    import bench

    path = bench.hip_runtime_path()
    assert os.path.basename(path).startswith("libamdhip64.so") and os.path.exists(path)
    assert bench.hip_event_flag("hipEventDisableSystemFence", 0) == 0x20000000
    assert bench.hip_event_flag("noSuchFlagAnywhere", 7) == 7


def _write_pass(d, counters, dispatches):
    """A rocprofv3 --pmc output directory: one CSV row per dispatch and counter."""
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
            "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
            "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
            "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    import csv
    with open(os.path.join(d, "host", "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(cols)
        for i, (name, grid, wg, vals) in enumerate(dispatches):
            for c in counters:
                w.writerow([i + 1, i + 1, "Agent 1", 1, 1, 1, grid, 1, name, wg, 0, 0, 8, 0, 16,
                            c, vals[c], 0, 1])


def test_counter_summary_attributes_dispatches_to_the_manifest(tmp_path):
    """The counter summary splits the library's dispatches into the manifest's items (runs of
    one kernel), calibrates on the copy probe and reports bytes against algorithmic bytes."""
    import json

    sys.path.insert(0, ROOT)
    import bench

    lib = "void mxfp8::(anonymous namespace)::{}(Args)"
    amax = lib.format("amax_vec_kernel<unsigned short, true, false, 2>")
    comb = lib.format("combine_kernel<unsigned short>")
    cast = lib.format("cast_vec_kernel<unsigned short, true, false, false, 2, false>")
    fill = "void at::native::vectorized_elementwise_kernel<16, FillFunctor<float> >(int)"
    copy = "__amd_rocclr_copyBuffer"
    kib = (256 << 20) / 1024
    man = {"argv": ["--steps", "1", "--counter-pass", "x.json"], "dtype": "bf16",
           "fused": False, "kernel_source_sha256_16": "0123456789abcdef",
           "copy_probe": {"launches": 24, "read_bytes": 256 << 20, "write_bytes": 256 << 20},
           "items": [{"label": "step_amax", "calls": 1, "alg_bytes": 1000 * 1024},
                     {"label": "step_combine", "calls": 1, "alg_bytes": 100 * 1024},
                     {"label": "step_cast", "calls": 1, "alg_bytes": 2000 * 1024},
                     {"label": "step_amax", "calls": 1, "alg_bytes": 1000 * 1024},
                     {"label": "step_combine", "calls": 1, "alg_bytes": 100 * 1024},
                     {"label": "step_cast", "calls": 1, "alg_bytes": 2000 * 1024},
                     {"label": "cast_bf16_full", "calls": 2, "alg_bytes": 4000 * 1024}]}
    # FETCH_SIZE reads half the bytes (a factor of 2, like gfx950's 64-byte units)
    step = [(fill, 4, 256, 50, 10), (amax, 100, 256, 900, 100), (comb, 10, 256, 80, 20),
            (cast, 100, 256, 1000, 1000)]
    disp = []
    for _ in range(2):
        disp += step
    disp += [(copy, 131072, 512, kib / 2, kib)] * 24
    # the table's set-up copy right behind the probe, of the same launch shape
    disp += [(copy, 131072, 512, kib / 4, kib / 2)]
    # two calls of two launches each (two buckets)
    disp += [(cast, 50, 256, 1000, 1000), (cast, 50, 256, 1000, 1000)] * 2
    for k, ctr, idx in (("fetch", "FETCH_SIZE", 3), ("write", "WRITE_SIZE", 4)):
        _write_pass(str(tmp_path / f"r_{k}"), [ctr],
                    [(d[0], d[1], d[2], {ctr: d[idx]}) for d in disp])
        json.dump(man, open(tmp_path / f"r_{k}.json", "w"))
    out = tmp_path / "s.md"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-counters",
                        str(tmp_path / "r"), "--out", str(out)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    block = json.loads(text.split("```json\n")[1].split("\n```")[0])
    assert block["fetch_factor"] == 2.0 and block["write_factor"] == 1.0
    per = block["hbm_bytes_per_launch"]
    assert per["step_amax"] == (2 * 900 + 100) * 1024
    assert per["step_cast"] == (2 * 1000 + 1000) * 1024
    # per launch = per call / launches per call
    assert per["cast_bf16_full"] == (2 * 2000 + 2000) * 1024 // 2
    assert "| cast_bf16_full | `cast_vec_kernel<bf16, true, false, false, 2, false>` | 2 | 2 |" \
        in text
    assert "--counter-pass $R/gpurun_out/cnt/r_fetch.json" in text
    assert " 1.9000 |" in text  # step_amax: (1800 + 100) KiB / 1000 KiB


def test_counter_summary_refuses_a_manifest_that_does_not_match(tmp_path):
    import json

    lib = "void mxfp8::(anonymous namespace)::amax_vec_kernel<float, true>(Args)"
    man = {"argv": ["--counter-pass", "x"], "dtype": "fp32", "fused": False,
           "kernel_source_sha256_16": "0", "copy_probe": {"launches": 1, "read_bytes": 1024,
                                                          "write_bytes": 1024},
           "items": [{"label": "step_amax", "calls": 1, "alg_bytes": 1},
                     {"label": "step_cast", "calls": 1, "alg_bytes": 1}]}
    for k, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        _write_pass(str(tmp_path / f"r_{k}"), [ctr], [(lib, 1, 256, {ctr: 1.0}),
                                                       ("__amd_rocclr_copyBuffer", 1, 1,
                                                        {ctr: 1.0})])
        json.dump(man, open(tmp_path / f"r_{k}.json", "w"))
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-counters",
                        str(tmp_path / "r")], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "1 runs of library launches, 2 manifest items" in r.stderr


def test_roofline_traffic_is_read_per_step_configuration(tmp_path, monkeypatch):
    """roofline.traffic comes from the summary of the same step (dtype, fused) taken on the
    current kernel source, and is null otherwise."""
    import json

    sys.path.insert(0, ROOT)
    import bench

    sha = bench.kernel_sha()
    for name, dt, fu, v in (("a", "bf16", False, 11), ("b", "fp32", False, 22),
                            ("c", "bf16", True, 33)):
        blk = {"dtype": dt, "fused": fu, "kernel_source_sha256_16": sha,
               "hbm_bytes_per_launch": {"step_cast" if not fu else "step_scales_cast": v}}
        (tmp_path / f"{name}_counters.md").write_text(
            "# x\n\n```json\n" + json.dumps(blk) + "\n```\n")
    old = {"dtype": "fp32", "fused": True, "kernel_source_sha256_16": "stale",
           "hbm_bytes_per_launch": {"step_scales_cast": 44}}
    (tmp_path / "d_counters.md").write_text("```json\n" + json.dumps(old) + "\n```\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.traffic_from_counters("bf16", False, "step_cast") == 11
    assert bench.traffic_from_counters("fp32", False, "step_cast") == 22
    assert bench.traffic_from_counters("bf16", True, "step_scales_cast") == 33
    assert bench.traffic_from_counters("fp32", True, "step_scales_cast") is None
