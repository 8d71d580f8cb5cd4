"""Handoff-latency analysis of the time journal on hand-built records (host logic, no GPU)."""
import numpy as np
import pytest

from decode_megakernel_wave_amd import synclat


def rec(cta, step, pc, op, t_wait, ready_rel, done_rel, xcc=0):
    return [cta, step, pc, op, t_wait & 0xFFFFFFFF, ready_rel, done_rel, xcc]


def test_handoff_latency_of_waiting_and_late_consumers():
    base = 0xFFFFFF00  # the 32-bit clock wraps inside the journal
    r = [
        # stage pc 0 (up_gate, op 5): three producers, the last one done at base + 100
        rec(0, 0, 0, 5, base, 5, 60),
        rec(1, 0, 0, 5, base, 5, 100),
        rec(2, 0, 0, 5, base, 5, 80),
        # stage pc 1 (down, op 6): two consumers waiting since before base + 100, one arriving late
        rec(0, 0, 1, 6, base + 60, 70, 200),    # ready at +130: latency 30 ticks
        rec(1, 0, 1, 6, base + 100, 50, 200),   # waits from +100 (== last done): ready +150, latency 50
        rec(2, 0, 1, 6, base + 120, 8, 200),    # started after the data was complete: 8 ticks of staging
        [0] * 8,                                # unused record
    ]
    res = synclat.handoffs(np.array(r, dtype=np.uint32))
    d = res["down"]
    assert d["waiting_consumers"] == 2 and d["stages"] == 1
    assert d["median_us"] == pytest.approx(0.40)           # median of 30 and 50 ticks
    assert d["critical_median_us"] == pytest.approx(0.50)  # last ready (+150) - last done (+100)
    assert d["late_staging_median_us"] == pytest.approx(0.08)
    assert d["span_median_us"] == pytest.approx(2.20)  # last consumer done (+320) - last producer done (+100)
    assert "up_gate" not in res  # the first stage of the journal has no producer in it
    assert res["all"]["waiting_consumers"] == 2


def test_records_without_a_staging_mark_are_skipped():
    r = [rec(0, 0, 0, 7, 1000, 5, 50), rec(0, 0, 1, 8, 1050, 0, 20), rec(0, 1, 0, 1, 1075, 10, 40)]
    res = synclat.handoffs(np.array(r, dtype=np.uint32))
    assert "argmax" not in res
    # the step after the argmax starts from a token every workgroup computed itself: a span, no handoff
    assert res["qkv"]["waiting_consumers"] == 0 and res["qkv"]["late_staging_median_us"] is None
    assert res["qkv"]["span_median_us"] == pytest.approx(0.45)  # 1075 + 40 - (1050 + 20)


def test_consumers_staged_before_the_last_producer_are_not_handoffs():
    r = [rec(0, 0, 0, 1, 0, 5, 100), rec(1, 0, 0, 1, 0, 5, 300),     # QKV producers: last done at 300
         rec(0, 0, 1, 2, 100, 50, 400),                               # needs only the early producer: ready 150
         rec(1, 0, 1, 2, 300, 40, 400)]                               # waits for the last: ready 340
    res = synclat.handoffs(np.array(r, dtype=np.uint32))
    a = res["attention"]
    assert a["waiting_consumers"] == 1 and a["median_us"] == pytest.approx(0.40)


def recp(cta, step, pc, op, t_wait, ready_rel, done_rel, pub_rel, xcc=0):
    """A record of the current layout: op | xcc << 24 | 1 << 31, publish time in the last word."""
    return [cta, step, pc, op | (xcc << 24) | (1 << 31), t_wait & 0xFFFFFFFF, ready_rel, done_rel, pub_rel]


def test_publish_time_is_the_handoff_start():
    """With a publish time in the record the latency runs from the last producer's publish (its
    stores issued), not from its done time after the failure vote; consumers staged before that
    publish are counted as early, not timed."""
    r = [recp(0, 0, 0, 4, 0, 5, 100, 70, xcc=3),   # O-proj producer: published at 70, done at 100
         recp(1, 0, 0, 4, 0, 5, 160, 130, xcc=5),  # the last producer: published at 130, done at 160
         recp(0, 0, 1, 5, 90, 60, 300, 280),       # waiting from 90: ready at 150 -> 20 ticks after 130
         recp(1, 0, 1, 5, 110, 70, 300, 280),      # waiting from 110: ready at 180 -> 50 ticks
         recp(2, 0, 1, 5, 20, 100, 300, 280)]      # ready at 120, before the last publish: early
    res = synclat.handoffs(np.array(r, dtype=np.uint32))
    u = res["up_gate"]
    assert u["waiting_consumers"] == 2 and u["early_consumers"] == 1
    assert u["median_us"] == pytest.approx(0.35)           # median of 20 and 50 ticks
    assert u["critical_median_us"] == pytest.approx(0.50)  # last ready (180) - last publish (130)
    assert u["span_median_us"] == pytest.approx(2.50)      # last consumer done (110 + 300) - last producer done (160)
    # op and xcc share a word: the op is still read from the low byte
    assert "o_proj" not in res and set(res) == {"up_gate", "all"}


def test_empty_journal():
    assert synclat.handoffs(np.zeros((4, 8), dtype=np.uint32)) == {}


def test_fine_marks_phase_medians():
    """Phases are differences of the marks of each instruction (10 ns ticks -> µs), medians per
    op over workgroups and instructions, unrecorded marks (0) left out, skipped indices ignored."""
    ts = np.zeros((3, 3, 8), dtype=np.uint64)
    for g in range(3):
        for i in range(3):
            t0 = 1000 * (i + 1) + 10 * g
            # marks in time order 0, 1, 2, 5, 7, 6, 3, 4 (array index = mark number)
            m = {0: t0, 1: t0 + 100 + g, 2: t0 + 110 + g, 5: t0 + 150 + g, 7: t0 + 200 + g,
                 6: t0 + 250 + g, 3: t0 + 300 + g, 4: t0 + 400 + g}
            for k, v in m.items():
                ts[g, i, k] = v
    ts[0, 0] = 1  # instruction 0 is skipped: its values must not count
    ts[2, 1, 4] = 0  # the vote mark of one instruction was not recorded
    res = synclat.fine_marks(ts, [None, "a", "a"])
    assert list(res) == ["a"]
    a = res["a"]
    assert a["wait_and_poll"] == pytest.approx(1.01)  # 100 + g over g = 0, 1, 2
    assert a["barrier"] == pytest.approx(0.10)
    assert a["activations"] == pytest.approx(0.40)
    assert a["first_chunk"] == pytest.approx(0.50)
    assert a["own_rows"] == pytest.approx(0.50)
    assert a["workgroup_and_publish"] == pytest.approx(0.50)
    assert a["vote"] == pytest.approx(1.00)
    assert a["total"] == pytest.approx(4.01)  # 400 + g without the unrecorded one: median of 5 values
