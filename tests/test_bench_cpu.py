"""bench.py contract checks that need no GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    # one GPU only: the cross-rank exchange is emulated on one device
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_step_bytes_counts_every_swap_and_the_roll():
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    w = workloads.make("full")
    swap, roll, total = bench.step_bytes(w, w.layers)
    assert swap == 2 * w.total * w.row_bytes
    j = w.max_shift
    assert roll == w.total * (8 + 8 * j + (j + 1))     # ids in; J shifted streams and J + 1 masks out
    assert total == 2 * w.layers * swap + roll


def test_timing_events_resolve_the_hip_runtime_through_the_library():
    # the bench's timing-only events call the HIP runtime the library is
    # linked against; resolving the four entry points needs no GPU
    sys.path.insert(0, ROOT)
    import bench
    hip = bench.TimingEvent._runtime()
    for name in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventElapsedTime", "hipEventDestroy"):
        assert getattr(hip, name) is not None
    assert bench.HIP_EVENT_DISABLE_SYSTEM_FENCE == 0x20000000
