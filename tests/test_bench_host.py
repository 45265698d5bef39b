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
