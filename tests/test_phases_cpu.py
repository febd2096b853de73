"""Host logic of the phase-log summary (no GPU): a synthetic log with known times."""
import pytest

from dense_matrix_unit_tiled_amd import profiling


def rec(start, loop, fix, end, clk0, clk1, xcc, wg, kt):
    return [start, loop, fix, end, clk0, clk1, xcc << 32, wg | (kt << 32)]


def test_phase_summary_known_log():
    # ticks of the 100 MHz clock: 1 tick = 0.01 us; two workgroups on XCDs 0 and 1
    log = [rec(1000, 1000 + 5000, 1000 + 5000, 1000 + 5500, 0, 2_200_000 * 55 // 1000, 0, 0, 64),
           rec(1100, 1100 + 6000, 1100 + 6000, 1100 + 6400, 0, 2_000_000 * 64 // 1000, 1, 1, 64)]
    s = profiling.phase_summary(log, 1, compute_units=4, launch_us=70.0)
    assert s["records"] == 2 and s["kind"] == "one workgroup per tile"
    assert s["span_us"] == pytest.approx(65.0)          # 1000 -> 7500 ticks
    assert s["start_skew_us"] == pytest.approx(1.0)
    assert s["main_loop_us"] == {"min": 50.0, "median": 55.0, "max": 60.0}
    assert s["epilogue_us"]["min"] == pytest.approx(4.0) and s["epilogue_us"]["max"] == pytest.approx(5.0)
    assert s["partial_sums_us"]["max"] == 0.0
    assert s["cu_time_covered"] == pytest.approx((55 + 64) / (4 * 65), abs=1e-4)
    assert s["shader_clock_ghz"]["min"] == pytest.approx(2.0, abs=1e-3)
    assert s["shader_clock_ghz"]["max"] == pytest.approx(2.2, abs=1e-3)
    assert s["records_per_xcd"] == {0: 1, 1: 1}
    assert s["per_xcd"][0]["main_loop_median_us"] == pytest.approx(50.0)
    assert s["per_xcd"][1]["end_max_us"] == pytest.approx(65.0)
    assert s["per_xcd"][1]["shader_clock_ghz_median"] == pytest.approx(2.0, abs=1e-3)
    assert s["outside_span_us"] == pytest.approx(5.0)
    text = profiling.phase_markdown("w", "k", "python3 bench.py --workload c3 --phases 20", s)
    assert "| main loop" in text and "65.00 µs" in text


def test_median_launch_is_the_recorded_one():
    mk = lambda span, keep: dict({"event_us": span, "kind": 1, "n": 1, "span_ticks": span},
                                 **({"records": [rec(0, 1, 1, span, 0, 1, 0, 0, 1)]} if keep else {}))
    raw = {"launches": [mk(300, False), mk(100, False), mk(200, True)], "median_launch": 2}
    assert profiling.median_launch(raw)["event_us"] == 200


def test_empty_log_rejected():
    with pytest.raises(ValueError):
        profiling.phase_summary([], 1, 4)
