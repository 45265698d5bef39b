"""Host-side pieces of bench.py (no GPU): the split launch count it reports
and the committed HBM byte counters it reads."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_attention_launches_of_a_split_call():
    # 3510 queries x 40 heads: 560 units, 48 left after two rounds of 256,
    # each cut into 5 key parts -> whole rounds, remainder, merge
    assert bench.attention_launches(3510, 40) == 3
    # 1800 queries: 320 units, 64 left in 4 parts
    assert bench.attention_launches(1800, 40) == 3
    # 2560 queries: 400 units, 144 left, one part each -> no merge launch
    assert bench.attention_launches(2560, 40) == 2


def test_measured_traffic_reads_the_committed_counters():
    # None when the summary is missing or the kernel source changed since the
    # counters were taken; else the scaled FETCH + WRITE bytes of one launch,
    # which can only exceed the 503 MB the 512x512 attention must move
    v = bench.measured_traffic("prsink_512")
    assert v is None or v > 503316480
    assert bench.measured_traffic("no_such_workload") is None


def _cpu_legs(name, **over):
    import torch
    from bounded_kv_block_amd import synth
    cfg = synth.workload(name, **over)
    poses = synth.poses(cfg, cfg["blocks"])

    def run_inputs(layer, block, step):
        return tuple(torch.from_numpy(a) for a in synth.qkv(cfg, layer, block, step))
    m = bench.steady_block(cfg) + 1
    return cfg, bench.cpu_baseline(cfg, run_inputs, poses, m, 0.05)


def test_cpu_baseline_legs_on_small_streams():
    # the oracle leg and the fp32 numpy leg both report whole-block query
    # tokens/s; a block of several attends (layers x steps) divides by them
    for name, over in (("tiny_fp32", {}),
                       ("prsink_720x416", dict(heads=2, grid_h=4, grid_w=5, layers=2, steps=3, pose_dim=8)),
                       ("convkv_512", dict(heads=2, grid_h=4, grid_w=4, blocks=10))):
        cfg, res = _cpu_legs(name, **over)
        assert res["kind"] == "oracle" and res["value"] > 0 and res["cores"] >= 1
        assert res["fp32_numpy"]["value"] > 0
        if cfg["layers"] * cfg["steps"] > 1:
            assert "attends per block" in res["sample"]


def test_more_than_one_gpu_exits_with_a_message():
    # the benchmark measures one GPU's share; N > 1 is refused before any GPU work
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                                     "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
