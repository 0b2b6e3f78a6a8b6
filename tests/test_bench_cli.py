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
