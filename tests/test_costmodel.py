"""The round cost model (lossy_kv_draft_amd.costmodel) against schedules worked out by
hand and against closed forms: the slot ring's critical path in the limiting cases,
the geometric acceptance sum by enumeration, and its inverse."""
import itertools

import numpy as np
import pytest

from lossy_kv_draft_amd import costmodel as CM


def C(**kw):
    base = dict(layers=4, slots=2, t_step=1.0, t_layer=2.0, t_stage=3.0, t_tail=0.5)
    base.update(kw)
    return CM.RoundCosts(**base)


def test_round_time_by_hand():
    # 4 layers, 2 slots, k = 2: drafts end at 2.  Copies: L0 [0,3], L1 [3,6]; verify L0
    # [3,5], L1 [6,8]; L2's slot frees at 5 (L0 verified) but the copy stream is busy
    # until 6: L2 [6,9], verify [9,11]; L3 waits for L1's verify (8): [9,12], verify
    # [12,14]; + tail 0.5
    assert CM.round_time(2, C()) == pytest.approx(14.5)
    # one slot per layer: copies back to back [0,3] .. [9,12]; verify of L3 ends at 14
    assert CM.round_time(2, C(slots=4)) == pytest.approx(14.5)
    # long drafts dominate: 10 steps, all staging under them, then 4 verified layers
    assert CM.round_time(10, C(slots=4)) == pytest.approx(10 + 4 * 2 + 0.5)


def test_round_time_limits():
    # an infinitely fast link: drafts then the verify pass, whatever the slots
    for R in (1, 2, 4):
        assert CM.round_time(8, C(t_stage=0.0, slots=R)) == pytest.approx(8 + 4 * 2 + 0.5)
    # a slow link with one slot: staging and verifying alternate layer by layer
    assert CM.round_time(1, C(slots=1, t_stage=10.0)) == pytest.approx(4 * (10 + 2) + 0.5)
    # the round never gets shorter when the link slows or the slots shrink
    ks = (1, 4, 16, 32)
    for k in ks:
        for R in (1, 2, 3, 4):
            times = [CM.round_time(k, C(slots=R, t_stage=s)) for s in (0.0, 0.5, 1.0, 4.0, 16.0)]
            assert all(a <= b + 1e-12 for a, b in zip(times, times[1:]))
        per_slots = [CM.round_time(k, C(slots=R)) for R in (1, 2, 3, 4)]
        assert all(a >= b - 1e-12 for a, b in zip(per_slots, per_slots[1:]))


def test_expected_commits_by_enumeration():
    """E[min(a + 1, k)] with P(a >= i) = p^i, enumerated over the accepted count a."""
    for p in (0.0, 0.3, 0.5, 0.9, 0.99):
        for k in (1, 2, 5, 32):
            probs = [p ** a * (1 - p) for a in range(k)] + [p ** k]        # a = 0..k-1, then all k accepted
            e = sum(pr * min(a + 1, k) for a, pr in enumerate(probs))
            assert CM.expected_commits(p, k) == pytest.approx(e, rel=1e-12, abs=1e-12)
    assert CM.expected_commits(1.0, 7) == 7.0


def test_accept_p_inverts_expected_commits():
    for k in (4, 32):
        for p in (0.05, 0.35, 0.8, 0.97):
            c = CM.expected_commits(p, k)
            assert CM.accept_p_from_commits(c, k) == pytest.approx(p, abs=1e-9)


def test_best_horizon_and_speedup_surface():
    costs = lambda k: C(t_layer=2.0 + 0.01 * k)
    # with every draft accepted the longest horizon wins; with none, the shortest
    assert CM.best_horizon(4, (4, 8, 16, 32), 1.0, costs) == 32
    assert CM.best_horizon(4, (4, 8, 16, 32), 0.0, costs) == 4
    rows = CM.speedup_surface(4, 32, C(), 100.0, 8.0, accepted_lens=(0.0, 10.0, 31.0), link_rates=(10.0, 100.0))
    assert len(rows) == 6
    by = {(a, r): x for a, r, _, x in rows}
    # more accepted drafts, or a slower link (staging dominates both), help draft-and-verify
    assert by[(31.0, 10.0)] > by[(10.0, 10.0)] > by[(0.0, 10.0)]
    assert by[(31.0, 10.0)] > by[(31.0, 100.0)]
