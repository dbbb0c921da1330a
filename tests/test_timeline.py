"""The per-wave timeline summary (mamba_selective_ssm_amd/timeline.py) on
synthetic stamp rows: the parser must recover each wave's pass, role, events
and clock, and the summary must report the phase durations the rows encode."""
import statistics

from mamba_selective_ssm_amd import timeline as tl


def _row(full, math, wv, seg, unit, rt0, events, ticks_per_us=2000.0):
    """One wave's row: entry realtime/memtime, header, (code, us) events, exit."""
    t0 = 10_000_000
    r = [0] * tl.SLOTS
    r[0] = rt0
    r[1] = t0
    r[2] = (int(full) << 63) | (int(math) << 62) | (wv << 48) | (seg << 32) | unit
    for i, (code, us) in enumerate(events):
        r[3 + i] = (code << 56) | (t0 + int(round(us * ticks_per_us)))
    end_us = events[-1][1] + 1.0
    r[tl.SLOTS - 2] = t0 + int(round(end_us * ticks_per_us))
    r[tl.SLOTS - 1] = rt0 + int(round(end_us * tl.REALTIME_MHZ))
    return r


def test_parse_header_and_events():
    ev = [(5, 0.2), (1, 1.0), (2, 1.5), (3, 4.0), (4, 4.5)]
    rows = [_row(True, False, 6, 3, 17, 1000, ev), [0] * tl.SLOTS]
    waves = tl.parse(rows)
    assert len(waves) == 1                     # the empty row (a wave that never ran) is skipped
    w = waves[0]
    assert (w["full"], w["math"], w["wv"], w["seg"], w["unit"]) == (True, False, 6, 3, 17)
    assert [c for c, _ in w["ev"]] == [5, 1, 2, 3, 4]
    assert abs(w["ev"][3][1] / 2000.0 - 4.0) < 1e-3


def test_summary_reports_encoded_phase_times():
    # two prep waves and one matrix-core wave of an output pass, three chunks each
    prep_steps = [(10, 0.0), (17, 0.1), (18, 0.4), (11, 0.6), (12, 0.7), (13, 0.9), (14, 1.2), (15, 2.0),
                  (16, 2.5)]
    def prep_events(offset):
        ev = [(5, 0.2), (1, 1.0), (2, 1.6), (3, 4.0), (4, 4.5)]
        t = 4.5
        for _ in range(3):
            ev += [(c, t + d) for c, d in prep_steps]
            t += 2.5
        return ev
    math_events = [(5, 0.3), (20, 1.0), (21, 1.2), (4, 4.5)]
    t = 4.5
    for _ in range(3):
        math_events += [(22, t + 1.5), (23, t + 2.0), (24, t + 2.2), (16, t + 2.5)]
        t += 2.5
    rows = [_row(True, False, 4, 0, 0, 500, prep_events(0)),
            _row(True, False, 5, 0, 0, 510, prep_events(0)),
            _row(True, True, 0, 0, 0, 505, math_events)]
    text = tl.summarize(tl.parse(rows), "synthetic")
    assert "2000 ticks per us" in text
    lines = text.splitlines()

    def row_value(label):
        hits = [l for l in lines if l.startswith("| " + label + " |")]
        assert hits, label
        return float(hits[0].split("|")[2])

    assert abs(row_value("rotation of B, C + next loads") - 0.8) < 0.02
    assert abs(row_value("phase C (outputs)") - 1.5) < 0.02
    assert abs(row_value("phase D (state update)") - 0.5) < 0.02
    assert abs(row_value("first loads issued") - 1.0) < 0.02
    # per-wave line: work before the barrier is prep start..rotation = 2.0 us, wait 0.5 us
    per = [l for l in lines if l.startswith("by wave index") and "w4" in l][0]
    assert "w4 2.00/0.50" in per and "w5 2.00/0.50" in per
