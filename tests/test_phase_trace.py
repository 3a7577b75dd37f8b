"""Host logic of the per-phase trace reader: spans between the marks of a call
are read from the right columns (no GPU; timestamps are synthetic)."""
import numpy as np

from causal_draft_correction_amd import phase_trace as pt


def _stamps(nblk, cols, per_block_skew=0):
    t = np.zeros((nblk, pt.SLOTS), np.int64)
    for b in range(nblk):
        for c, v in cols.items():
            t[b, c] = v + b * per_block_skew
    return t


def test_resident_spans():
    K = 4
    cols = {}
    # prologue: start 0, loads issued at 1 us, anchor step 2..5 us, prologue end 6 us
    for s, us in ((511, 0), (508, 1), (-16, 2), (-12, 5), (509, 6)):
        cols[s + pt.RES_BIAS] = int(us / pt.TICK_US)
    # position p starts at 10 + 10 p us; marks k us later for slot 32 p + k
    for p in range(K):
        for k in (0, 1, 2, 4, 5, 13, 16, 18, 19, 20):
            cols[32 * p + k + pt.RES_BIAS] = int((10 + 10 * p + 0.25 * k) / pt.TICK_US)
    r = pt.summarize(_stamps(3, cols), K, batched=False)
    assert r["prologue"]["anchor_step"] == [3.0, 3.0]
    assert r["prologue"]["prologue"] == [6.0, 6.0]
    mid = r["positions_1_to_2_median"]
    assert mid["argmax_exchange"] == [2.0, 2.0]  # marks 5 -> 13
    assert mid["position"] == [10.0, 10.0]
    assert mid["u_hop"] == [5.0, 5.0]  # mark 20 of p -> mark 0 of p + 1
    assert "state_dots" not in r["position_3"]  # the last position has no state step
    assert abs(r["kernel_us"] - (10 + 30 + 0.25 * 13)) <= 0.05


def test_batched_spans_and_slowest_block():
    K = 3
    cols = {1019: 0, 1023: 100, 1022: 150, 1021: 200, 1020: 300}
    for p in range(K):
        for k in (0, 7, 1, 2, 3, 4, 5):
            cols[64 * p + k] = 1000 + 2000 * p + 100 * [0, 7, 1, 2, 3, 4, 5].index(k)
    r = pt.summarize(_stamps(5, cols, per_block_skew=0), K, batched=True)
    assert r["prologue"]["w2_slice_load"] == [1.0, 1.0]
    assert r["positions_1_to_1_median"]["w2"] == [1.0, 1.0]
    assert r["positions_1_to_1_median"]["position"] == [20.0, 20.0]
    # one slow block shows in the max column only
    t = _stamps(5, cols)
    t[2, 64 + 1] += 500
    r = pt.summarize(t, K, batched=True)
    assert r["positions_1_to_1_median"]["w2"] == [1.0, 6.0]
