"""Host-side parts of bench.py and the counter folding (no GPU)."""
import os
import subprocess
import sys

from draft_verification_softmax_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _csv(path, rows):
    hdr = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,Kernel_Id,Kernel_Name,"
           "Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,Accum_VGPR_Count,SGPR_Count,Counter_Name,"
           "Counter_Value,Start_Timestamp,End_Timestamp\n")
    with open(path, "w") as f:
        f.write(hdr)
        for d, name, counter, val in rows:
            f.write(f'{d},{d},"Agent 1",1,1,1,1,1,"{name}",256,0,0,0,0,0,"{counter}",{val},0,1\n')


def test_traffic_calibration(tmp_path):
    # copy kernel: 1 GiB read shows as 524288 FETCH units and 1048576 WRITE units
    _csv(tmp_path / "cf.csv", [(1, "neg_kernel", "FETCH_SIZE", 524288.0), (2, "neg_kernel", "FETCH_SIZE", 524288.0)])
    _csv(tmp_path / "cw.csv", [(1, "neg_kernel", "WRITE_SIZE", 1048576.0)])
    # two dispatches of the kernel under test, one counter row split over two instances
    _csv(tmp_path / "f.csv", [(5, "sv::stream_kernel<1>", "FETCH_SIZE", 1000.0),
                              (5, "sv::stream_kernel<1>", "FETCH_SIZE", 24.0),
                              (6, "sv::stream_kernel<1>", "FETCH_SIZE", 1024.0)])
    _csv(tmp_path / "w.csv", [(5, "sv::stream_kernel<1>", "WRITE_SIZE", 10.0)])
    t = profiling.traffic(tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "cf.csv", tmp_path / "cw.csv",
                          1 << 30, ["stream_kernel"], copy_match="neg")
    assert t["fetch_scale"] == 2048.0 and t["write_scale"] == 1024.0
    assert t["stream_kernel"]["fetch_bytes"] == 1024 * 2048.0
    assert t["stream_kernel"]["write_bytes"] == 10 * 1024.0
    assert t["stream_kernel"]["dispatches"] == 2


def test_launch_percentiles():
    """p10 / median / p90 of the per-launch times: nearest rank on the sorted times, in us."""
    import bench

    t = bench.Timed(None, None)
    t.per_launch_ms = [0.1 + 0.001 * i for i in range(401)][::-1]   # 100..500 us, unsorted
    assert t.percentiles_us() == {"p10": 140.0, "p50": 300.0, "p90": 460.0}
    t.per_launch_ms = [0.25]
    assert t.percentiles_us() == {"p10": 250.0, "p50": 250.0, "p90": 250.0}
