"""Whole rounds of the tiny fp32 head at its exact workload shape (hidden 256,
4/2 heads, head_dim 64, intermediate 768, vocabulary 1024, a 128-slot draft KV
prefix, two drafts per round, greedy), launched as the benchmark launches them,
against the oracle round by round (see ``compare_rounds``).

The literal workload draws N(0, 3) target logits per round: random weights make
nearly every draft a rejection, so those 64 rounds exercise the one-pair
flushes.  A second run plants acceptance with p_i = 0.8 * 0.85^i (the depth
workload's rule) under both KV policies, so the two- and three-pair flushes,
the kept chain entries of policy B and the bonus token run as well."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mtp_draft_head_step_amd import inputs as I
from tests.gpu_util import build, compare_rounds, kv_pair

pytestmark = pytest.mark.gpu

PREFIX, N = 128, 2


def _session(wl):
    shape = I.TINY_F32
    _, gh, oh = build(shape, wl)
    gkv, okv = kv_pair(shape, wl, PREFIX, PREFIX + 2 * 64 * (N + 1) + 8)
    committed = I.tokens_uniform(wl, 1, PREFIX + 2, shape.vocab)
    hid0 = I.target_hiddens(shape, wl, 1000, 1)[0]
    return shape, gh, oh, gkv, okv, committed, hid0


@pytest.mark.timeout(300)
def test_tiny_rounds_literal():
    shape, gh, oh, gkv, okv, committed, hid0 = _session(I.WL_TINY)

    def targets(rnd, drafts):
        return (I.logits_rows(I.WL_TINY, 5, rnd, N + 1, shape.vocab, 3.0)[0],
                I.target_hiddens(shape, I.WL_TINY, rnd, N + 1))

    ks, near = compare_rounds(gh, oh, gkv, okv, shape, committed, hid0, N, targets, 64)
    assert len(ks) == 64 and near <= 2


@pytest.mark.timeout(300)
@pytest.mark.parametrize("policy", ["A", "B"])
def test_tiny_rounds_planted(policy):
    shape, gh, oh, gkv, okv, committed, hid0 = _session(I.WL_TINY + 100)
    plan = [I.acceptance_draws(I.WL_TINY, (500, r), N) for r in range(32)]

    def targets(rnd, drafts):
        rows = I.logits_rows(I.WL_TINY, 5, (501, rnd), N + 1, shape.vocab, 3.0)[0]
        I.plant_acceptance(rows, np.asarray(drafts, np.int64), plan[rnd])
        return rows, I.target_hiddens(shape, I.WL_TINY, (502, rnd), N + 1)

    ks, near = compare_rounds(gh, oh, gkv, okv, shape, committed, hid0, N, targets, len(plan), policy=policy)
    assert ks == plan and set(ks) == {0, 1, 2} and near <= 2
