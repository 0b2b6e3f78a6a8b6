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


MARK = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<short> >(int)"
LIB = "void mxfp8::(anonymous namespace)::{}(Args)"
AMAX = LIB.format("amax_vec_kernel<unsigned short, true, false, 2>")
AMAX_ROW = LIB.format("amax_vec_kernel<unsigned short, false, false, 2>")
COMB = LIB.format("combine_kernel<unsigned short>")
CAST = LIB.format("cast_vec_kernel<unsigned short, true, false, false, 2, false>")
FILL = "void at::native::vectorized_elementwise_kernel<16, FillFunctor<float> >(int)"
COPY = "__amd_rocclr_copyBuffer"
KIB = (256 << 20) / 1024


def _manifest(items):
    return {"argv": ["--steps", "1", "--counter-pass", "x.json"], "dtype": "bf16",
            "fused": False, "kernel_source_sha256_16": "0123456789abcdef",
            "copy_probe": {"launches": 24, "read_bytes": 256 << 20, "write_bytes": 256 << 20},
            "items": items}


def _synthetic_run():
    """A manifest and its dispatches (name, grid, workgroup, FETCH KiB, WRITE KiB, µs): two
    steps, the copy probe, a table entry of two calls of two launches each and a layer-batch
    stage whose call runs two kernels."""
    items = []
    disp = [(MARK, 1, 256, 0, 0, 1.0)]  # the marker tensor's zero-fill
    for _ in range(2):
        disp.append((FILL, 4, 256, 50, 10, 1.0))  # the step's zero-fill: not an item
        for label, kern, alg, f, w, us in (("step_amax", AMAX, 1000, 900, 100, 30.0),
                                           ("step_combine", COMB, 100, 80, 20, 5.0),
                                           ("step_cast", CAST, 2000, 1000, 1000, 70.0)):
            items.append({"label": label, "calls": 1, "alg_bytes": alg * 1024})
            disp += [(MARK, 1, 256, 0, 0, 1.0), (kern, 100, 256, f, w, us)]
    items.append({"label": "copy_probe", "calls": 1, "alg_bytes": 2 * (256 << 20)})
    disp += [(MARK, 1, 256, 0, 0, 1.0)] + [(COPY, 131072, 512, KIB / 2, KIB, 100.0)] * 24
    items.append({"label": "cast_bf16_full", "calls": 2, "alg_bytes": 4000 * 1024})
    # the table's set-up copy and fill land in the previous span: not library launches
    disp += [(COPY, 131072, 512, KIB / 4, KIB / 2, 50.0), (FILL, 4, 256, 1, 1, 1.0),
             (MARK, 1, 256, 0, 0, 1.0)]
    disp += [(CAST, 50, 256, 1000, 1000, 10.0), (CAST, 50, 256, 1000, 1000, 12.0)] * 2
    # an aux item (a check between measured items): it only delimits
    items.append({"label": "abl_check_x", "calls": 1, "alg_bytes": 0, "aux": True})
    disp += [(MARK, 1, 256, 0, 0, 1.0), (CAST, 50, 256, 7, 7, 3.0), (AMAX, 60, 256, 7, 7, 3.0)]
    items.append({"label": "layer_k_buffers_amax", "calls": 1, "alg_bytes": 3000 * 1024})
    disp += [(MARK, 1, 256, 0, 0, 1.0), (AMAX, 60, 256, 1500, 50, 20.0),
             (AMAX_ROW, 40, 256, 1000, 30, 15.0)]
    return _manifest(items), disp


def _write_trace(d, dispatches):
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    cols = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
            "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
            "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X",
            "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    import csv
    t = 1000000
    with open(os.path.join(d, "host", "p_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(cols)
        for i, (name, grid, wg, us) in enumerate(dispatches):
            w.writerow(["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, i + 1, 1, name, i + 1, t,
                        t + int(us * 1000), 0, 0, 8, 0, 16, wg, 1, 1, grid, 1, 1])
            t += int(us * 1000) + 500


def test_counter_summary_attributes_dispatches_to_the_manifest(tmp_path):
    """The counter summary splits the dispatches at the markers into the manifest's items,
    calibrates on the copy probe and reports bytes against algorithmic bytes."""
    import json

    man, disp = _synthetic_run()
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
    assert per["layer_k_buffers_amax"] == (2 * 2500 + 80) * 1024 // 2
    assert "copy_probe" not in per and "abl_check_x" not in per
    assert "| cast_bf16_full | `cast_vec_kernel<bf16, true, false, false, 2, false>` | 2 | 2 |" \
        in text
    assert ("| layer_k_buffers_amax | `amax_vec_kernel<bf16, true, false, 2>`, "
            "`amax_vec_kernel<bf16, false, false, 2>` | 2 | 1 |") in text
    assert "--counter-pass $R/gpurun_out/cnt/r_fetch.json" in text
    assert " 1.9000 |" in text  # step_amax: (1800 + 100) KiB / 1000 KiB


def test_trace_summary_reports_kernel_time_per_call(tmp_path):
    import json

    man, disp = _synthetic_run()
    _write_trace(str(tmp_path / "r_trace"), [(d[0], d[1], d[2], d[5]) for d in disp])
    json.dump(man, open(tmp_path / "r_trace.json", "w"))
    out = tmp_path / "t.md"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-trace",
                        str(tmp_path / "r"), "--out", str(out)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    row = [l for l in text.splitlines() if l.startswith("| cast_bf16_full |")][0].split("|")
    assert row[3].strip() == "2" and row[4].strip() == "2"
    assert float(row[5]) == 22.0  # each call: 10 + 12 µs
    amax = [l for l in text.splitlines() if l.startswith("| step_amax |")][0].split("|")
    assert float(amax[5]) == 30.0 and amax[4].strip() == "2"
    assert float(amax[9]) == round(1000 * 1024 / 30e-6 / 1e9, 1)
    layer = [l for l in text.splitlines() if l.startswith("| layer_k_buffers_amax |")][0]
    assert "| 35.00 |" in layer
    assert "median of 24 launches: 100.00 µs" in text
    assert "abl_check_x" not in text
    assert "--kernel-trace --stats" in text


def test_counter_summary_refuses_a_manifest_that_does_not_match(tmp_path):
    import json

    man, disp = _synthetic_run()
    man["items"] = man["items"][:-1]  # one item fewer than the marked spans
    for k, ctr, idx in (("fetch", "FETCH_SIZE", 3), ("write", "WRITE_SIZE", 4)):
        _write_pass(str(tmp_path / f"r_{k}"), [ctr],
                    [(d[0], d[1], d[2], {ctr: d[idx]}) for d in disp])
        json.dump(man, open(tmp_path / f"r_{k}.json", "w"))
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-counters",
                        str(tmp_path / "r")], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "10 marked spans, 9 manifest items" in r.stderr


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
    # a running library built from another kernel source gets no counter traffic
    assert bench.traffic_from_counters("bf16", False, "step_cast", sha) == 11
    assert bench.traffic_from_counters("bf16", False, "step_cast", "0123456789abcdef") is None


def test_kernel_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench

    src = open(bench.KERNEL_SRC).read()
    base = bench.kernel_sha()
    f = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "KERNEL_SRC", str(f))
    f.write_text(src.replace("// ", "//  note: ", 3) + "\n/* a new\n   comment */\n")
    assert bench.kernel_sha() == base
    f.write_text(src.replace("kBlockLen", "kBlockLen + 0", 1))
    assert bench.kernel_sha() != base


def test_stats_summary_reads_the_kernel_stats_and_the_bench_line(tmp_path):
    import csv
    import json

    d = tmp_path / "step_bf16"
    os.makedirs(d / "host")
    with open(d / "host" / "step_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                    "StdDev"])
        w.writerow([CAST, 10, 730000, 73000.0, 50.0, 70000, 76000, 1.0])
        w.writerow([AMAX, 10, 360000, 36000.0, 25.0, 35000, 37000, 1.0])
        w.writerow([FILL, 11, 88000, 8000.0, 5.0, 7000, 9000, 1.0])
    line = {"dtype": "bf16", "steps": 200, "warmup": 1000,
            "config": {"rows": 16384, "cols": 6144, "workload": "a step"},
            "roofline": {"kernel": "cast_vec_kernel<bf16, colwise>", "launch_us": 73.1,
                         "launch_us_with_dispatch": 75.0, "alg_bytes_per_launch": 408944694},
            "stage_us_breakdown_pass": {"cast": 74.0}, "graph_us_per_step": 141.0}
    (tmp_path / "step_bf16.log").write_text("noise\n" + json.dumps(line) + "\n")
    out = tmp_path / "s.md"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-stats",
                        str(d), "--out", str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    assert "| `cast_vec_kernel<bf16, true, false, false, 2, false>` | 10 | 73.00 | 70.00 | 76.00 |" \
        in text
    assert "in 73.00 µs on average = 5.60 TB/s (70.0% of 8 TB/s)" in text
    # the benchmark's command, rebuilt from the sections its JSON line lacks
    assert ("python -u $R/bench.py --no-kernel-table --no-cpu-baseline --no-single-pass "
            "--no-layer-batch > $R/gpurun_out/stats/step_bf16.log 2>&1") in text
