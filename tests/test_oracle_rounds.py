"""Pins for the oracle's round driver: the temperature-0 exactness gate (MTP output
equals classic decode), the S/S+1 pairing through a from-scratch rebuild of the
draft KV, rollback leaving the prefix untouched, policy B bookkeeping, block size
and planted acceptance statistics.  CPU only."""
import math

import numpy as np
import pytest

from mtp_draft_head_step_amd import inputs as I
from oracle import head as H
from oracle import rounds as R
from oracle.kvcache import DraftKV, ROUND_BASE
from oracle.verify import Sampling

SHAPE = I.HeadShape(hidden=64, n_q_heads=2, n_kv_heads=1, head_dim=32, intermediate=128, vocab=64)
L0 = 6           # synthetic prefix length
CAP = 160


def random_head(seed=21):
    return H.Head(SHAPE, I.weight_values(SHAPE, I.head_weights(SHAPE, seed)))


def successor_head(seed=22):
    """A head whose greedy draft is (look-ahead token + 1) mod V: fc = [I | 0],
    o_proj = 0, down_proj = 0 (so g = x = RMSNorm(E[t])), lm_head row j = E[j - 1]."""
    w = I.weight_values(SHAPE, I.head_weights(SHAPE, seed))
    h = SHAPE.hidden
    w["fc"] = np.zeros((h, 2 * h), np.float32)
    w["fc"][:, :h] = np.eye(h)
    w["o_proj"] = np.zeros_like(w["o_proj"])
    w["down_proj"] = np.zeros_like(w["down_proj"])
    for n in I.NORM_TENSORS:
        w[n] = np.ones_like(w[n])
    e = np.random.default_rng(seed).standard_normal((SHAPE.vocab, h)).astype(np.float32)
    w["embed"] = e
    w["lm_head"] = np.roll(e, 1, axis=0)
    return H.Head(SHAPE, w)


def session(head, tgt, prompt_len=L0 + 2):
    """A session whose prompt was prefilled: prompt tokens, prefix KV for slots
    [0, L0) (synthetic), and the remaining completed pairs pending."""
    r = np.random.default_rng(5)
    committed = [int(t) for t in r.integers(0, SHAPE.vocab, prompt_len)]
    kp, vp = I.prefix_kv(SHAPE, 9, L0, CAP)
    kv = DraftKV(1, CAP, 32, kp, vp, L0)
    pending = [(committed[s + 1], tgt.hidden_state(committed[s], s)) for s in range(L0, prompt_len - 1)]
    return R.RoundState(head, kv, pending, committed, window=16), (kp, vp)


def target_fn_of(tgt):
    return lambda toks, start: tgt.forward(toks, start)


@pytest.mark.parametrize("policy", ["A", "B"])
@pytest.mark.parametrize("n_draft", [1, 2, 3])
@pytest.mark.parametrize("headkind", ["random", "successor"])
def test_exactness_gate_greedy_equals_classic(policy, n_draft, headkind):
    """Temperature 0: the MTP stream is byte-identical to classic greedy decode."""
    head = random_head() if headkind == "random" else successor_head()
    tgt = I.ToyTarget(31, SHAPE.vocab, SHAPE.hidden, follow=0.8 if headkind == "successor" else 0.0)
    st, _ = session(head, tgt)
    start = list(st.committed)
    ks = []
    for _ in range(14):
        out = R.run_round(st, n_draft, target_fn_of(tgt), policy=policy)
        assert st.invariant()
        assert 1 <= len(out["tokens"]) <= n_draft + 1          # committed per round <= block_size
        ks.append(out["k"])
    classic = R.classic_greedy(target_fn_of(tgt), start, len(st.committed) - len(start))
    assert st.committed == classic
    if headkind == "successor":
        assert max(ks) == n_draft and min(ks) == 0              # full and partial acceptance occurred
    assert st.kv.err == 0


@pytest.mark.parametrize("n_draft", [2, 3])
def test_policy_a_kv_equals_from_scratch_flush(n_draft):
    """Policy A: after every round the draft KV on [0, len) equals a from-scratch
    flush of the committed pairs (t_{S+1}, h_S) on top of the synthetic prefix."""
    head = successor_head()
    tgt = I.ToyTarget(32, SHAPE.vocab, SHAPE.hidden, follow=0.7)
    st, (kp, vp) = session(head, tgt)
    template = DraftKV(1, CAP, 32, kp, vp, L0)
    for _ in range(10):
        R.run_round(st, n_draft, target_fn_of(tgt), policy="A")
        c = st.committed
        pairs = R.pairs_from_stream(c, lambda s: tgt.hidden_state(c[s], s), L0, st.kv.len)
        ref = R.rebuild_kv(head, template, pairs, L0)
        n = st.kv.len
        assert np.array_equal(st.kv.K[:, :n], ref.K[:, :n]) and np.array_equal(st.kv.V[:, :n], ref.V[:, :n])
    # a planted pairing mistake (h_S paired with t_S) does not reproduce the cache
    bad = [(c[s], tgt.hidden_state(c[s], s)) for s in range(L0, st.kv.len)]
    refb = R.rebuild_kv(head, template, bad, L0)
    assert not np.array_equal(st.kv.K[:, L0:st.kv.len], refb.K[:, L0:st.kv.len])


def test_policy_b_keeps_accepted_chain_entries():
    head = successor_head()
    tgt = I.ToyTarget(33, SHAPE.vocab, SHAPE.hidden, follow=0.9)
    st, _ = session(head, tgt)
    n_draft = 3
    seen = set()
    for _ in range(12):
        before_len = st.kv.len + len(st.pending)                 # = round base after the flush
        out = R.run_round(st, n_draft, target_fn_of(tgt), policy="B")
        k = out["k"]
        keep = min(k, n_draft - 1)
        assert st.kv.len == before_len + keep
        assert len(st.pending) == k + 1 - keep
        assert st.invariant()
        seen.add(k)
    assert 0 in seen and n_draft in seen


def test_rollback_keeps_prefix_bytes():
    head = random_head()
    kp, vp = I.prefix_kv(SHAPE, 9, L0, CAP)
    kv = DraftKV(1, CAP, 32, kp, vp, L0)
    r = np.random.default_rng(3)
    head.flush(kv, [1, 2, 3], [r.standard_normal(64) for _ in range(3)], H.LAST, set_round_base=True)
    head.step(kv, 4, r.standard_normal(64))
    head.step(kv, 5, r.standard_normal(64))
    snapK, snapV = kv.K.copy(), kv.V.copy()
    assert kv.len == L0 + 5 and kv.base == L0 + 3
    kv.rollback(ROUND_BASE)                                      # policy A
    assert kv.len == L0 + 3
    assert np.array_equal(kv.K, snapK) and np.array_equal(kv.V, snapV)   # no byte changes at all
    kv.rollback(L0 + 1)
    assert kv.len == L0 + 1
    kv.rollback(L0 + 2)                                          # beyond the length: sticky error
    assert kv.err != 0 and kv.len == L0 + 1
    kv.rollback(0)
    assert kv.len == L0 + 1                                      # no-op after the error


def test_rollback_skipped_breaks_kv_equality():
    """The mutation the pages ask a test for: leaving the rolled-back state
    un-restored must be detected.  Skipping the rollback leaves provisional chained
    entries in the cache, which then differs from the from-scratch rebuild."""
    head = random_head()
    tgt = I.ToyTarget(34, SHAPE.vocab, SHAPE.hidden)
    st, (kp, vp) = session(head, tgt)
    st.kv.rollback = lambda *a, **k: None                       # planted mistake, oracle side
    R.run_round(st, 3, target_fn_of(tgt), policy="A")
    R.run_round(st, 3, target_fn_of(tgt), policy="A")
    c = st.committed
    n = len(c) - 1 - len(st.pending)                           # where the cache should end
    pairs = R.pairs_from_stream(c, lambda s: tgt.hidden_state(c[s], s), L0, n)
    ref = R.rebuild_kv(head, DraftKV(1, CAP, 32, kp, vp, L0), pairs, L0)
    assert st.kv.len != n or not np.array_equal(st.kv.K[:, :n], ref.K[:, :n])


def test_block_size_is_drafts_plus_one():
    """block_size = mtp_depth + 2 with depth 1 gives block_size 3 = 2 drafts + the
    bonus: the verify covers N + 1 = 3 target rows."""
    mtp_depth = 1
    block_size = mtp_depth + 2
    n_draft = block_size - 1
    head = random_head()
    tgt = I.ToyTarget(35, SHAPE.vocab, SHAPE.hidden)
    st, _ = session(head, tgt)
    seen_rows = []
    out = R.run_round(st, n_draft, lambda toks, s: (seen_rows.append(len(toks)), tgt.forward(toks, s))[1])
    assert n_draft == 2 and len(out["drafts"]) == 2 and seen_rows == [block_size]


def test_planted_acceptance_closed_form():
    """Acceptance drawn per position with p_i = 0.8 * 0.85^i: the mean committed per
    round matches 1 + sum_j prod_{i<j} p_i (1.8, 2.344, 2.6584, ... for N = 1, 2, 3)."""
    want = [1.8, 2.344, 2.6584, 2.8129, 2.8774, 2.9003, 2.9072, 2.9090]
    rounds = 3000
    for n in range(1, 9):
        exact = 1 + sum(math.prod(0.8 * 0.85 ** i for i in range(j)) for j in range(1, n + 1))
        assert abs(exact - want[n - 1]) < 6e-4
        ks = np.array([I.acceptance_draws(5, (n, r), n) for r in range(rounds)])
        mean = (ks + 1).mean()
        sd = (ks + 1).std()
        assert abs(mean - exact) < 4 * sd / math.sqrt(rounds) + 1e-9


def test_planted_rows_give_planted_k():
    from oracle.verify import verify
    r = np.random.default_rng(4)
    for trial in range(20):
        n = int(r.integers(1, 9))
        k = int(r.integers(0, n + 1))
        rows = r.standard_normal((n + 1, 500)).astype(np.float32) * 3
        d = r.integers(0, 500, n).astype(np.int64)
        I.plant_acceptance(rows, d, k)
        out = verify(Sampling(), rows, None, list(d), np.zeros(4, np.int32), np.array([0, 0], np.int32))
        assert out["k"] == k and out["tokens"][:k] == [int(t) for t in d[:k]]


@pytest.mark.parametrize("policy", ["A", "B"])
def test_batch_ragged_acceptance_equals_classic_per_session(policy):
    """B = 3 sessions with different prompt lengths, targets and head behaviour
    (two follow their successor heads' drafts with different rates, one never
    does), driven together round by round: acceptance is ragged (the sessions'
    k differ within rounds), every session's committed stream is its own classic
    greedy decode, and every session keeps its own invariant
    kv.len + pending = committed - 1."""
    from oracle import batch as Bt
    head = successor_head()
    tgts = [I.ToyTarget(40 + b, SHAPE.vocab, SHAPE.hidden, follow=f) for b, f in enumerate([0.9, 0.5, 0.0])]
    states, starts = [], []
    for b, tgt in enumerate(tgts):
        st, _ = session(head, tgt, prompt_len=L0 + 2 + b)
        states.append(st)
        starts.append(list(st.committed))
    fns = [target_fn_of(t) for t in tgts]
    ragged = 0
    for _ in range(10):
        outs = Bt.run_batch_round(states, 3, fns, policy=policy)
        ks = [o["k"] for o in outs]
        ragged += len(set(ks)) > 1
        assert all(st.invariant() for st in states)
    assert ragged >= 3
    for st, start, fn in zip(states, starts, fns):
        assert st.committed == R.classic_greedy(fn, start, len(st.committed) - len(start))
    assert len({st.kv.len for st in states}) > 1          # the sessions sit at different lengths
