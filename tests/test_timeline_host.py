"""Host logic of the timeline tool: launch grouping and the per-launch and
whole-call summaries, on hand-made records with known answers."""
import numpy as np

from gram_newton_schulz_amd import timeline


def _rec(t0, t1, t2, t3, cu, K, grid, mode=0, queue=0, cycles=None):
    r = np.zeros(8, dtype=np.uint64)
    r[0], r[1], r[2], r[3] = t0, t1, t2, t3
    # shader cycles: 20 per 10 ns tick of the 100 MHz clock, i.e. 2 GHz
    r[4] = cycles if cycles is not None else 20 * (t3 - t0)
    r[6] = K | (grid << 32) | (mode << 56)
    hw = (cu & 0x7F) << 8 | (queue & 7) << 24
    r[7] = hw
    return r


def test_two_launches_on_two_cus():
    recs = [
        # launch A (K=4096, 4 workgroups on 2 CUs): two rounds
        _rec(0, 10, 110, 120, cu=0, K=4096, grid=4),
        _rec(0, 10, 110, 120, cu=1, K=4096, grid=4),
        _rec(120, 130, 230, 240, cu=0, K=4096, grid=4),
        _rec(120, 130, 180, 190, cu=1, K=4096, grid=4),
        # launch B (same kind and grid, starts after A has ended)
        _rec(300, 310, 410, 420, cu=0, K=4096, grid=4),
        _rec(300, 310, 410, 420, cu=1, K=4096, grid=4),
        _rec(420, 430, 530, 540, cu=0, K=4096, grid=4),
        _rec(420, 430, 530, 540, cu=1, K=4096, grid=4),
    ]
    s = timeline.summarize(np.stack(recs))
    L = s["launches"]
    assert len(L) == 2
    a, b = L
    assert a["workgroups"] == 4 and a["K"] == 4096 and a["kind"] == "sym"
    assert abs(a["span_us"] - 2.4) < 1e-9                   # 240 ticks of 10 ns
    assert abs(a["prologue_us"] - 0.1) < 1e-9
    assert abs(a["loop_us"] - (100 + 100 + 100 + 50) / 4 * 0.01) < 1e-9
    assert abs(a["epilogue_us"] - 0.1) < 1e-9
    # CU 1 idles 50 ticks at the tail, CU 0 none
    assert abs(a["tail_idle_us"] - 0.25) < 1e-9
    assert abs(a["busy_frac"] - (120 * 3 + 70) / (2 * 240)) < 1e-12
    assert abs(b["start_us"] - 3.0) < 1e-9
    assert abs(a["clock_ghz"] - 2.0) < 1e-9
    c = s["call"]
    assert c["cus"] == 2 and c["workgroups"] == 8
    fr = c["cu_time_frac"]
    assert abs(sum(fr.values()) - 1.0) < 1e-12
    assert abs(fr["idle"] - (2 * 540 - (120 * 3 + 70) - 4 * 120) / (2 * 540)) < 1e-12


def test_streams_are_separated_by_queue():
    # two concurrent launches of the same kind on two queues, interleaved in
    # record order, must not merge
    recs = []
    for k in range(4):
        recs.append(_rec(10 * k, 10 * k + 5, 10 * k + 50, 10 * k + 60, cu=k, K=16384, grid=4, queue=0))
        recs.append(_rec(10 * k + 2, 10 * k + 7, 10 * k + 52, 10 * k + 62, cu=4 + k, K=16384, grid=4, queue=1))
    s = timeline.summarize(np.stack(recs))
    assert [x["workgroups"] for x in s["launches"]] == [4, 4]


def test_kind_change_starts_a_new_launch():
    recs = [_rec(0, 1, 2, 3, cu=0, K=4096, grid=2), _rec(0, 1, 2, 3, cu=1, K=4096, grid=2),
            _rec(1, 2, 3, 4, cu=0, K=4096, grid=2, mode=2), _rec(1, 2, 3, 4, cu=1, K=4096, grid=2, mode=2)]
    s = timeline.summarize(np.stack(recs))
    assert [x["kind"] for x in s["launches"]] == ["sym", "final"]
