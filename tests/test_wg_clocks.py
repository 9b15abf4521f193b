"""CPU tests of the per-work-group clock summariser (decode_attention_03_amd/wg_clocks.py):
its figures, on synthetic stamps whose answers are known, and its --from-raw path.
The stamps are what the instrumented balanced kernel writes per work-group: start and
end ticks of the 100 MHz clock, pieces, K/V tokens, and the word holding the XCD in
bits 24..31 above the block index."""
import json
import math
import sys

import pytest

from decode_attention_03_amd import wg_clocks, workloads

TICK_US = 1e6 / wg_clocks.CLOCK_HZ  # 0.01 us per tick


def _stamp(start, end, pieces, tokens, xcd, block):
    return (start, end, pieces, tokens, (xcd << 24) | block)


def test_span_busy_fraction_and_rates():
    row = 512  # bytes of K + V per token of one KV head (d = 128, 16-bit)
    # launch 0: two work-groups, the second starts 1 us late and ends 4 us later
    a = [_stamp(1000, 11000, 1, 1000, 0, 0), _stamp(1100, 15000, 2, 2000, 1, 1)]
    # launch 1: the same shape, shifted in time (times are taken per launch)
    b = [_stamp(50000, 60000, 1, 1000, 0, 0), _stamp(50100, 64000, 2, 2000, 1, 1)]
    r = wg_clocks.analyse([a, b], row)
    assert r["launches"] == 2 and r["work_groups"] == 2
    span = (15000 - 1000) * TICK_US  # 140 us
    assert math.isclose(r["span_us"]["median"], span)
    assert math.isclose(r["span_us"]["min"], span) and math.isclose(r["span_us"]["max"], span)
    busy = ((11000 - 1000) + (15000 - 1100)) * TICK_US / (2 * span)
    assert math.isclose(r["mean_busy_frac"], busy)
    assert math.isclose(r["start_us"][0], 0.0) and math.isclose(r["start_us"][100], 1.0)
    assert math.isclose(r["finish_us"][0], 100.0) and math.isclose(r["finish_us"][100], 140.0)
    # rates: tokens * row bytes / duration
    r0 = 1000 * row / (100e-6) / 1e9
    r1 = 2000 * row / (139e-6) / 1e9
    assert math.isclose(r["rate_GBps"][0], min(r0, r1))
    assert math.isclose(r["rate_GBps"][100], max(r0, r1))
    assert set(r["rate_by_xcd_GBps"]) == {0, 1}
    assert math.isclose(r["rate_by_xcd_GBps"][0], r0)
    assert math.isclose(r["rate_by_xcd_GBps"][1], r1)


def test_percentiles_pick_order_statistics():
    # 101 work-groups ending at 0, 1, ..., 100 us after a common start
    wgs = [_stamp(0, 100 * i, 1, 10, i % 8, i) for i in range(1, 102)]
    r = wg_clocks.analyse([wgs], 256)
    assert math.isclose(r["finish_us"][0], 1.0)
    assert math.isclose(r["finish_us"][50], 51.0)
    assert math.isclose(r["finish_us"][90], 91.0)
    assert math.isclose(r["finish_us"][100], 101.0)
    assert sorted(r["rate_by_xcd_GBps"]) == list(range(8))


def test_summary_file(tmp_path):
    wgs = [_stamp(0, 10000, 1, 100, 0, 0), _stamp(0, 12000, 1, 120, 3, 1)]
    res = {"workload": "w_test", "plan_work_groups": 4, **wg_clocks.analyse([wgs], 512)}
    path = wg_clocks.write_summary(res, 4, str(tmp_path / "out"))
    text = open(path, encoding="utf-8").read()
    assert path.endswith("wg_clocks_w_test.md")
    assert "2 of 4 work-groups had work" in text
    assert "| kernel span, first start to last end (µs) | median 120.0" in text
    assert "0: " in text and "3: " in text


def test_from_raw_matches_analyse(tmp_path, monkeypatch, capsys):
    w = workloads.WORKLOADS[4]
    launches = [[[0, 9000, 1, 4000, 2 << 24], [10, 9500, 2, 4100, (5 << 24) | 1]]]
    raw = tmp_path / "stamps.json"
    raw.write_text(json.dumps({"workload": w.name, "plan_work_groups": 2,
                               "launches": launches}))
    monkeypatch.setattr(sys, "argv", ["wg_clocks", "--config", "4", "--from-raw", str(raw)])
    assert wg_clocks.main() == 0
    printed = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    expect = wg_clocks.analyse([[tuple(x) for x in launches[0]]], w.head_dim * 2 * 2)
    assert printed["workload"] == w.name
    assert math.isclose(printed["span_us"]["median"], expect["span_us"]["median"])
    assert math.isclose(printed["mean_busy_frac"], expect["mean_busy_frac"])


def test_from_raw_refuses_other_workload(tmp_path, monkeypatch):
    raw = tmp_path / "stamps.json"
    raw.write_text(json.dumps({"workload": "something_else", "launches": [[[0, 1, 1, 1, 0]]]}))
    monkeypatch.setattr(sys, "argv", ["wg_clocks", "--config", "4", "--from-raw", str(raw)])
    with pytest.raises(SystemExit):
        wg_clocks.main()
