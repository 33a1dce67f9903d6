"""Oracle: the draft-depth controller.  TEST INFRASTRUCTURE ONLY.

The depth controller picks, for every round, how many tokens the head drafts.
It maximises committed tokens per unit of wall-clock time,

    N* = argmax_N committed(N) / cost(N),

from live per-position acceptance and a per-width round cost, with N = 0
(plain decode, nothing drafted) as the floor and N running up to one past the
acceptance frontier (the deepest position drafted so far).  Every
``interval`` rounds it drafts one deeper than its choice (a probe, so the
position past the frontier gets measured); the interval starts at 4 rounds and
backs off up to 512.  Its state (counts, cost table, cadence, choice) lives in
one object that persists across requests.

Sources: "Ollama qwen3_5 MTP loader and SelfDraft path", Facts on depth control
(the argmax of committed over cost from live per-position acceptance and
per-width forward cost, depth 0 as the floor, a probe past the choice every 4
rounds backing off to 512, state kept across requests), and the Ollama
x/mlxrunner commit log (the commit that chooses the speculative draft length to
maximise throughput, replacing a schedule that grew on acceptance alone).

Readings where the pages leave a step open (plainest choice, stated):
  * per-position acceptance a_i = P(draft i accepted | drafts 1..i-1 were),
    estimated with Laplace's rule (accepts_i + 1) / (attempts_i + 2), so an
    untried position counts as a coin flip;
  * committed(N) = 1 + sum_{i=1..N} prod_{j<=i} a_j: the correction or bonus
    token always commits, each accepted draft adds one, and a round stops at
    its first rejection;
  * cost(N) is the caller's per-width table (seconds or any unit, > 0) for a
    round drafting N tokens, seeded by the caller and updated from reported
    round times by an exponential average with weight 1/4 on the new time;
  * the frontier F is the deepest position with an attempt; candidates are
    N = 0 .. min(max_depth, F + 1); ties go to the smaller N;
  * probe cadence: a counter of rounds since the last probe; when it reaches
    the interval the round drafts min(choice + 1, max_depth) and the interval
    doubles (capped at 512); a change of choice resets the interval to 4.
"""
from __future__ import annotations

PROBE_FIRST = 4
PROBE_MAX = 512
COST_WEIGHT = 0.25


def acceptance(accepts: int, attempts: int) -> float:
    """Laplace estimate of one position's conditional acceptance."""
    return (accepts + 1.0) / (attempts + 2.0)


def committed(rates, n: int) -> float:
    """Expected committed tokens of a round drafting n tokens, given the
    per-position conditional acceptance rates (rates[0] is position 1)."""
    total, run = 1.0, 1.0
    for i in range(n):
        run = run * rates[i]
        total = total + run
    return total


class DepthController:
    def __init__(self, max_depth: int, cost):
        if max_depth < 0 or len(cost) != max_depth + 1 or any(not (c > 0) for c in cost):
            raise ValueError("depth controller: max_depth >= 0 and a positive cost per depth 0..max_depth")
        self.max_depth = max_depth
        self.cost = [float(c) for c in cost]
        self.attempts = [0] * (max_depth + 1)      # index i = position i (index 0 unused)
        self.accepts = [0] * (max_depth + 1)
        self.interval = PROBE_FIRST
        self.since_probe = 0
        self.choice = self._argmax()

    def rates(self):
        return [acceptance(self.accepts[i], self.attempts[i]) for i in range(1, self.max_depth + 1)]

    def frontier(self) -> int:
        f = 0
        for i in range(1, self.max_depth + 1):
            if self.attempts[i] > 0:
                f = i
        return f

    def _argmax(self) -> int:
        r = self.rates()
        top = min(self.max_depth, self.frontier() + 1)
        best, best_n = None, 0
        for n in range(top + 1):
            v = committed(r, n) / self.cost[n]
            if best is None or v > best:
                best, best_n = v, n
        return best_n

    def next_depth(self) -> int:
        """The depth to draft this round (a probe one past the choice when due)."""
        self.since_probe += 1
        if self.since_probe >= self.interval:
            self.since_probe = 0
            self.interval = min(2 * self.interval, PROBE_MAX)
            return min(self.choice + 1, self.max_depth)
        return self.choice

    def report(self, depth: int, accepted: int, round_cost: float) -> None:
        """A round drafted ``depth`` tokens, ``accepted`` of them were accepted,
        and it took ``round_cost``."""
        if not (0 <= depth <= self.max_depth and 0 <= accepted <= depth and round_cost > 0):
            raise ValueError("depth controller: report outside its range")
        for i in range(1, min(accepted + 1, depth) + 1):
            self.attempts[i] += 1
            if i <= accepted:
                self.accepts[i] += 1
        self.cost[depth] = (1.0 - COST_WEIGHT) * self.cost[depth] + COST_WEIGHT * round_cost
        new = self._argmax()
        if new != self.choice:
            self.choice = new
            self.interval = PROBE_FIRST
            self.since_probe = 0
