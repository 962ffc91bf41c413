"""Two-stage load/compute pipeline timing model (test infrastructure only).

[TMA-atlas] section "Science and assumptions": with N equal tiles, a
two-stage pipeline first pays one load and one compute, then N - 1 further
tile intervals, each as long as the slower of the two stages.  Without
overlap the same work costs N times (load + compute).  The model assumes
independent load and compute resources, enough buffering, equal tiles and
free synchronisation; shared bandwidth can shrink or erase the overlap.

Symbols follow that section: ``n`` tiles, ``t_load`` and ``t_compute`` per
tile, all times in the same unit.  Its "Engineering example" (4 tiles, 3 us
load, 5 us compute) is the test fixture ``tests/golden/pipeline_example.txt``.
"""


def _check(n, t_load, t_compute):
    if int(n) != n or n < 1:
        raise ValueError("n must be a positive integer tile count")
    if t_load < 0 or t_compute < 0:
        raise ValueError("stage times must be non-negative")


def serial_time(n, t_load, t_compute):
    """No overlap: every tile is loaded, then computed."""
    _check(n, t_load, t_compute)
    return n * (t_load + t_compute)


def pipelined_time(n, t_load, t_compute):
    """Fill (first load + first compute), then n - 1 intervals of the slower stage."""
    _check(n, t_load, t_compute)
    return t_load + t_compute + (n - 1) * max(t_load, t_compute)
