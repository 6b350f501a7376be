"""Host-side logic of bench.py (no GPU): the steps captured per HIP graph."""

import bench


def test_steps_per_graph_divides_the_timed_steps():
    for steps in range(1, 400):
        per = bench.steps_per_graph(steps)
        assert 1 <= per <= 8
        assert steps % per == 0
        # the largest such divisor
        assert all(steps % d for d in range(per + 1, min(8, steps) + 1))
    assert bench.steps_per_graph(200) == 8
    assert bench.steps_per_graph(100) == 5
    assert bench.steps_per_graph(13) == 1
