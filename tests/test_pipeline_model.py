"""Pins for the two-stage pipeline timing model: the worked example printed on
the "Tensor Memory Accelerator" atlas page ("Engineering example") and the
model's elementary properties."""

import os

import pytest

from oracle import pipelined_time, serial_time

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pipeline_example.txt")


def _rows():
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                yield [float(v) for v in line.split()]


def test_pages_worked_example():
    rows = list(_rows())
    assert rows
    for n, tl, tc, serial, piped in rows:
        assert serial_time(int(n), tl, tc) == serial
        assert pipelined_time(int(n), tl, tc) == piped


def test_single_tile_has_no_overlap():
    for tl, tc in [(3, 5), (0.5, 0.25), (0, 1)]:
        assert pipelined_time(1, tl, tc) == serial_time(1, tl, tc)


def test_properties():
    for n in range(1, 12):
        for tl in [0.0, 1.0, 2.5, 7.0]:
            for tc in [0.0, 1.0, 3.0]:
                p = pipelined_time(n, tl, tc)
                assert p <= serial_time(n, tl, tc)
                assert p == pipelined_time(n, tc, tl)  # symmetric in the two stages
                # steady state is set by the slower stage
                assert p >= n * max(tl, tc)
    # equal stages: overlap approaches a 2x gain
    assert serial_time(100, 1, 1) / pipelined_time(100, 1, 1) == pytest.approx(200 / 101)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        pipelined_time(0, 1, 1)
    with pytest.raises(ValueError):
        serial_time(2, -1, 1)
