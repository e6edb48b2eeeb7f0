"""The decode timeline tool's arithmetic on made-up timestamps (no GPU): times are microseconds
of the 100 MHz clock from the first workgroup's start, per-workgroup stream times and the
serial tail are read from the right slots, and launches without the in-kernel merge report
the stream part only."""
import numpy as np
import pytest

from block_sparse_long_phase1_amd import decode_timeline as dt


def _ticks(us):
    return np.uint64(round(us * 100))


def test_summary_of_a_merged_launch():
    base = 1_000_000.0   # the clock's origin is arbitrary
    t = np.zeros((dt.GROUPS, dt.SLOTS), dtype=np.uint64)
    # three workgroups: (start, stream end, stores done, ticket) in us after `base`
    rows = [(0.0, 20.0, 21.0, 21.5), (0.5, 22.5, 23.0, 23.25), (2.0, 21.0, 21.75, 22.0)]
    for i, (s, e, st, tk) in enumerate(rows):
        t[i, 0], t[i, 1], t[i, 2], t[i, 3] = (_ticks(base + x) for x in (s, e, st, tk))
    # tickets: workgroup 1 drew the last one and merges (past its acquire at +0.5 us, done at
    # +2.5 us); workgroup 2 still holds merge slots from an earlier launch, which must be ignored
    t[0, 6], t[1, 6], t[2, 6] = 0, 2, 1
    t[1, 4], t[1, 5] = _ticks(base + 23.75), _ticks(base + 25.75)
    t[2, 4], t[2, 5] = _ticks(base - 100.0), _ticks(base - 98.0)
    r = dt._summary(t, 3)
    assert r["workgroups"] == 3
    assert r["start_spread"] == pytest.approx(2.0)
    assert r["stream_median"] == pytest.approx(20.0)      # durations 20, 22, 19
    assert r["stream_max"] == pytest.approx(22.0)
    assert r["stream_end"] == pytest.approx(22.5)
    assert r["store_wait_median"] == pytest.approx(0.75)  # 1.0, 0.5, 0.75
    assert r["ticket_median"] == pytest.approx(0.25)      # 0.5, 0.25, 0.25
    assert r["last_ticket"] == pytest.approx(23.25)
    assert r["mergers"] == 1
    assert r["merge_acquire"] == pytest.approx(0.5)
    assert r["merge"] == pytest.approx(2.5)
    assert r["end"] == pytest.approx(25.75)


def test_summary_without_the_in_kernel_merge():
    t = np.zeros((dt.GROUPS, dt.SLOTS), dtype=np.uint64)
    for i, (s, e) in enumerate([(0.0, 10.0), (1.0, 12.0)]):
        t[i, 0], t[i, 1] = _ticks(50.0 + s), _ticks(50.0 + e)
    r = dt._summary(t, 2)
    assert r["stream_end"] == pytest.approx(12.0)
    assert r["stream_max"] == pytest.approx(11.0)
    assert "merge" not in r and "last_ticket" not in r


def test_table_takes_medians_per_workload_and_kind():
    rows = [{"config": "w", "mode": m, "event_us": v, "end": v - 1.0} for m, v in
            (("warm", 10.0), ("warm", 12.0), ("warm", 30.0), ("cold", 20.0))]
    text = dt.table(rows)
    assert "| w | warm | 12.00 |" in text and "| w | cold | 20.00 |" in text
