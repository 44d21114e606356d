"""Host logic of the timeline report (masked_gqa_attention_amd.timeline) on
hand-made records: the record check, the per-event statistics, the per-wave
steps between events and the per-XCD table.  No GPU."""
import numpy as np

from masked_gqa_attention_amd import timeline as T


def _record(xcd, times, hw=5):
    """One wave's record: times[e] in counter ticks (0: event not reached)."""
    rec = np.zeros(9, dtype=np.uint64)
    rec[0] = np.uint64(1 | (xcd << 4) | (hw << 32))
    rec[1:1 + len(times)] = times
    return rec


def test_check_records_finds_missing_and_decreasing():
    good = np.stack([_record(0, [100, 110, 120, 130, 140, 150, 160]), _record(1, [101, 0, 125, 140, 0, 0, 0])])
    assert T.check_records(good) == []
    missing = good.copy()
    missing[1, 0] = 0
    assert any("no record" in p for p in T.check_records(missing))
    backwards = good.copy()
    backwards[0, 3] = 105  # event 2 before event 1
    assert any("decrease" in p for p in T.check_records(backwards))


def test_summary_of_split_kernel_records():
    # Four waves on two XCDs; times in ticks of 10 ns.  Wave 3 is the last
    # arrival (event 7).
    recs = []
    for w in range(4):
        b = 1000 + 10 * w
        t = [b, b + 100, b + 300, b + 2000 + 100 * w, b + 2100 + 100 * w, b + 2150 + 100 * w, b + 2200 + 100 * w]
        if w == 3:
            t.append(b + 2400 + 100 * w)
        recs.append(_record(w % 2, t))
    s = T.summarise(np.stack(recs), "splitkv_kernel")
    assert s["waves"] == 4
    ev = {e["event"]: e for e in s["events"]}
    assert ev[0]["min"] == 0.0 and abs(ev[0]["max"] - 0.30) < 1e-9  # starts 0, 10, 20, 30 ticks
    assert ev[7]["waves"] == 1 and abs(ev[7]["max"] - (30 + 2400 + 300) * 0.01) < 1e-9
    # span: latest event of any wave, from the first start
    assert abs(s["span"] - (30 + 2400 + 300) * 0.01) < 1e-9
    steps = {(p["from"], p["to"]): p for p in s["phases"]}
    first = steps[(T.EVENTS["splitkv_kernel"][0], T.EVENTS["splitkv_kernel"][1])]
    assert first["waves"] == 4 and abs(first["median"] - 1.0) < 1e-9
    last = steps[(T.EVENTS["splitkv_kernel"][6], T.EVENTS["splitkv_kernel"][7])]
    assert last["waves"] == 1 and abs(last["median"] - 2.0) < 1e-9
    # per XCD: XCD 0 holds waves 0, 2; XCD 1 waves 1, 3 (loop end = event 3)
    x = {r["xcd"]: r for r in s["xcd"]}
    assert x[0]["waves"] == 2 and abs(x[0]["loop_end_median"] - np.median([20.0, 22.2])) < 1e-9
    assert abs(x[1]["last_end"] - 27.30) < 1e-9


def test_kernel_of_plans():
    assert T.kernel_of({"path": 1, "keys_per_tile": 256}, 128) == ("splitkv_kernel", 8)
    assert T.kernel_of({"path": 1, "keys_per_tile": 128}, 128) == ("splitkv_kernel", 4)
    assert T.kernel_of({"path": 2, "keys_per_tile": 96}, 72) == ("encoder_kernel", 8)
    assert T.kernel_of({"path": 0, "keys_per_tile": 32}, 128) == ("prefill_pipe4_kernel", 4)
    assert T.kernel_of({"path": 0, "keys_per_tile": 64}, 64) == ("prefill_kernel", 8)
    for name, events in T.EVENTS.items():
        assert len(events) == 8 and events[0] == "start" and T.LOOP_END[name] < 8
