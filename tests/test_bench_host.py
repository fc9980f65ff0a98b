"""Host-side rules of bench.py (no GPU): how many steps each captured HIP
graph holds, so that exactly --steps steps are timed."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_graph_size_divides_steps():
    for steps in range(1, 401):
        g = bench.graph_size(steps)
        assert 1 <= g <= 10 and steps % g == 0
        if steps % 2 == 0:
            # the largest even divisor up to 10
            assert g % 2 == 0 and all(steps % d for d in range(g + 2, 11, 2))
        else:
            assert all(steps % d for d in range(g + 1, 10))


def test_graph_size_examples():
    assert bench.graph_size(50) == 10      # the default --steps
    assert bench.graph_size(20) == 10
    assert bench.graph_size(16) == 8
    assert bench.graph_size(12) == 6
    assert bench.graph_size(25) == 5
    assert bench.graph_size(7) == 7
    assert bench.graph_size(11) == 1
