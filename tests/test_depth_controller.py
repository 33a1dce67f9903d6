"""The library's draft-depth controller (host code behind the C ABI) against
the oracle: the same seeded rounds give the same depth every round, the same
choice and probe interval, and bit-identical cost tables; bad arguments fail
closed.  Host-only calls: no GPU needed."""
import numpy as np
import pytest

from mtp_draft_head_step_amd import abi
from oracle import depth as D


def _run(max_depth, cost, p, noise, rounds, seed):
    nat = abi.DepthController(max_depth, cost)
    ora = D.DepthController(max_depth, cost)
    rng = np.random.default_rng(seed)
    for r in range(rounds):
        d = nat.next()
        assert d == ora.next_depth(), r
        k = 0
        while k < d and rng.uniform() < p[k]:
            k += 1
        t = cost[d] * (1.0 + noise * rng.standard_normal())
        t = max(t, 1e-3)
        nat.report(d, k, t)
        ora.report(d, k, t)
        ch, iv, c = nat.state()
        assert (ch, iv) == (ora.choice, ora.interval), r
        assert c == ora.cost, r
    return ora


@pytest.mark.parametrize("seed", range(4))
def test_matches_oracle_planted_acceptance(seed):
    """Acceptance 0.8 * 0.85^(i-1) per position, linear round cost with 3% noise."""
    m = 8
    p = [0.8 * 0.85 ** i for i in range(m)]
    cost = [1.0 + 0.35 * n for n in range(m + 1)]
    ora = _run(m, cost, p, 0.03, 3000, seed)
    assert 1 <= ora.choice <= m


def test_matches_oracle_steep_cost_prefers_plain_decode():
    m = 4
    p = [0.3] * m
    cost = [1.0, 2.0, 3.0, 4.0, 5.0]
    ora = _run(m, cost, p, 0.02, 600, 11)
    assert ora.choice == 0


def test_matches_oracle_measured_curve():
    """Costs shaped like the 27B-head round (flat up to a few drafts, then
    growing) and high acceptance."""
    m = 16
    cost = [0.46] + [0.46 + 0.44 * n + (0.01 * n * n if n > 4 else 0.0) for n in range(1, m + 1)]
    p = [0.95] * m
    _run(m, cost, p, 0.05, 2000, 5)


def test_rejects_bad_arguments():
    with pytest.raises(abi.MtpError):
        abi.DepthController(-1, [])
    with pytest.raises(abi.MtpError):
        abi.DepthController(17, [1.0] * 18)              # past MTP_MAX_DRAFT
    with pytest.raises(abi.MtpError):
        abi.DepthController(2, [1.0, 0.0, 1.0])
    with pytest.raises(abi.MtpError):
        abi.DepthController(2, [1.0, float("nan"), 1.0])
    c = abi.DepthController(2, [1.0, 1.5, 2.0])
    with pytest.raises(abi.MtpError):
        c.report(3, 0, 1.0)
    with pytest.raises(abi.MtpError):
        c.report(1, 2, 1.0)
    with pytest.raises(abi.MtpError):
        c.report(1, 0, 0.0)
    assert c.state()[0] == 0                           # 1.5 / 1.5 ties plain decode: the smaller wins
