"""Pins of the depth-controller oracle (oracle/depth.py) against what the
pages and the arithmetic fix: the expected committed count equals brute-force
enumeration of accept/reject outcomes, the choice is the argmax of committed
over cost (a hand example and brute force over random tables), plain decode
wins when drafts never pay, the probe cadence 4, 8, ..., 512, and the counting
of a round's report."""
import itertools

import numpy as np
import pytest

from oracle import depth as D


def enumerate_committed(rates, n):
    """E[1 + accepted] of a round drafting n tokens, by summing over every
    accept/reject sequence (a rejection ends the round)."""
    total = 0.0
    for outcome in itertools.product([0, 1], repeat=n):
        p, k, alive = 1.0, 0, True
        for i, acc in enumerate(outcome):
            if not alive:
                # positions after the first rejection are not drafted: count the
                # sequence once, with its trailing entries fixed to 0
                if acc:
                    p = 0.0
                continue
            p *= rates[i] if acc else (1.0 - rates[i])
            if acc:
                k += 1
            else:
                alive = False
        total += p * (1 + k)
    return total


@pytest.mark.parametrize("seed", range(6))
def test_committed_matches_enumeration(seed):
    r = np.random.default_rng(seed).uniform(0, 1, 7)
    for n in range(8):
        assert D.committed(r, n) == pytest.approx(enumerate_committed(r, n), rel=1e-12)


def test_committed_special_cases():
    assert D.committed([0.3, 0.9], 0) == 1.0
    assert D.committed([1.0] * 5, 5) == 6.0                  # every draft accepted
    assert D.committed([0.0, 1.0, 1.0], 3) == 1.0            # position 1 always rejected
    assert D.committed([0.5] * 3, 3) == pytest.approx(1 + 0.5 + 0.25 + 0.125)


def test_laplace_estimate():
    assert D.acceptance(0, 0) == 0.5
    assert D.acceptance(7, 8) == 0.8
    assert D.acceptance(0, 98) == pytest.approx(1 / 100)


def test_report_counts_positions():
    c = D.DepthController(3, [1.0, 1.0, 1.0, 1.0])
    c.report(3, 1, 1.0)                 # position 1 accepted, 2 rejected, 3 never drafted
    assert c.attempts[1:] == [1, 1, 0] and c.accepts[1:] == [1, 0, 0]
    c.report(3, 3, 1.0)                 # all three accepted
    assert c.attempts[1:] == [2, 2, 1] and c.accepts[1:] == [2, 1, 1]
    c.report(0, 0, 1.0)                 # plain decode: nothing drafted
    assert c.attempts[1:] == [2, 2, 1]
    c.report(2, 0, 1.0)
    assert c.attempts[1:] == [3, 2, 1] and c.accepts[1:] == [2, 1, 1]
    with pytest.raises(ValueError):
        c.report(2, 3, 1.0)
    with pytest.raises(ValueError):
        c.report(4, 0, 1.0)


def test_cost_moves_by_quarter_weight():
    c = D.DepthController(1, [2.0, 4.0])
    c.report(1, 0, 8.0)
    assert c.cost == [2.0, 5.0]
    c.report(0, 0, 6.0)
    assert c.cost == [3.0, 5.0]


def test_hand_example():
    """a1 = 8/10, a2 = 2/4 after these rounds; costs fixed at 1, 1.5, 1.9, 2.4:
    ratios 1, 1.8/1.5 = 1.2, 2.2/1.9 = 1.158, 2.4/2.4 = 1 (a3 untried: 1/2),
    so the choice is one draft."""
    cost = [1.0, 1.5, 1.9, 2.4]
    c = D.DepthController(3, cost)
    for d, k in [(2, 2), (2, 1)] + [(1, 1)] * 5 + [(1, 0)]:
        c.report(d, k, cost[d])                     # the average keeps these costs
    assert c.cost == cost
    assert c.rates()[:3] == [0.8, 0.5, 0.5]
    assert c.frontier() == 2
    assert c.choice == 1


def test_plain_decode_when_drafts_never_pay():
    c = D.DepthController(4, [1.0, 1.2, 1.4, 1.6, 1.8])
    for _ in range(50):
        c.report(1, 0, 1.2)
    assert c.choice == 0


def test_grows_one_past_the_frontier_when_drafts_always_pay():
    c = D.DepthController(8, [1.0] * 9)         # flat cost: deeper is never worse
    assert c.choice == 1                        # frontier 0: candidates 0..1
    for d in range(1, 9):
        c.report(d, d, 1.0)
        assert c.choice == min(d + 1, 8)


@pytest.mark.parametrize("seed", range(8))
def test_choice_is_brute_force_argmax(seed):
    rng = np.random.default_rng(100 + seed)
    m = 6
    cost = list(np.sort(rng.uniform(1.0, 3.0, m + 1)))
    c = D.DepthController(m, cost)
    for _ in range(40):
        d = int(rng.integers(0, m + 1))
        c.report(d, int(rng.integers(0, d + 1)), float(rng.uniform(1.0, 3.0)))
    rates = [(c.accepts[i] + 1) / (c.attempts[i] + 2) for i in range(1, m + 1)]
    deepest = max([i for i in range(1, m + 1) if c.attempts[i] > 0], default=0)
    cands = range(0, min(m, deepest + 1) + 1)
    vals = [enumerate_committed(rates, n) / c.cost[n] for n in cands]
    best = max(vals)
    assert c.choice == min(n for n, v in zip(cands, vals) if v >= best - 1e-12)


def test_probe_cadence_backs_off_to_512():
    c = D.DepthController(4, [1.0, 1.5, 2.0, 2.5, 3.0])
    assert c.choice == 0
    probes = [i for i in range(1, 4000) if c.next_depth() != 0]
    gaps = np.diff([0] + probes).tolist()
    assert gaps[:8] == [4, 8, 16, 32, 64, 128, 256, 512]
    assert set(gaps[8:]) == {512}


def test_probe_interval_resets_when_choice_changes():
    c = D.DepthController(2, [1.0, 1.2, 1.4])
    assert c.choice == 1                        # 1.5 / 1.2 > 1 with an untried position 1
    for _ in range(3):
        c.next_depth()
    assert c.next_depth() == c.choice + 1 and c.interval == 8
    before = c.choice
    for _ in range(20):
        c.report(1, 0, 1.2)                     # position 1 keeps failing
    assert c.choice != before and c.choice == 0
    assert c.interval == 4 and c.since_probe == 0


def test_converges_to_the_best_depth_under_planted_acceptance():
    """Acceptance p_i = 0.8 * 0.85^(i-1) per position and a linear round cost:
    the controller settles on the depth whose closed-form ratio is largest."""
    m = 8
    p = [0.8 * 0.85 ** i for i in range(m)]
    cost = [1.0 + 0.35 * n for n in range(m + 1)]
    truth = int(np.argmax([D.committed(p, n) / cost[n] for n in range(m + 1)]))
    c = D.DepthController(m, cost)
    rng = np.random.default_rng(7)
    for _ in range(4000):
        d = c.next_depth()
        k = 0
        while k < d and rng.uniform() < p[k]:
            k += 1
        c.report(d, k, cost[d])
    assert c.choice == truth
