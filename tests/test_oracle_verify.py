"""Pins for the oracle's sampler transform and speculative verification:
hand-worked examples, library special cases, and an exact brute-force check that
rejection sampling reproduces sequential sampling from the target.  CPU only."""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import verify as Vf
from oracle.verify import Sampling


def test_penalize_hand_example():
    x = np.array([2.0, -2.0, 1.0, 0.0], np.float32)
    y = Vf.penalize(x, [0, 1, 1, 3], 2.0)          # token 1 counted once; 0 stays 0
    assert y.tolist() == [1.0, -4.0, 1.0, 0.0]


def test_plain_softmax_special_case():
    x = np.random.default_rng(0).standard_normal(50).astype(np.float32) * 3
    ids, p, _ = Vf.transform(x, [], Sampling(temperature=1.0))
    assert ids.tolist() == list(range(50))
    assert np.allclose(p, softmax(x.astype(np.float64)), atol=1e-14)


def test_top_k_one_is_argmax_lowest_id():
    x = np.array([1.0, 5.0, 5.0, 2.0], np.float32)
    ids, p, _ = Vf.transform(x, [], Sampling(temperature=0.8, top_k=1))
    assert ids.tolist() == [1] and p.tolist() == [1.0]


def test_hand_worked_top_p_min_p_temperature():
    # probabilities 1/2, 1/4, 1/8, 1/8
    x = np.log(np.array([4.0, 2.0, 1.0, 1.0])).astype(np.float32)
    ids, p, info = Vf.transform(x, [], Sampling(temperature=1.0, top_p=0.7))
    assert ids.tolist() == [0, 1] and np.allclose(p, [2 / 3, 1 / 3], atol=1e-7)
    assert abs(info["top_p_margin"] - 0.05) < 1e-6                 # 0.75 - 0.7
    ids, p, _ = Vf.transform(x, [], Sampling(temperature=1.0, min_p=0.3))
    assert ids.tolist() == [0, 1]                                  # 0.25/0.5 kept, 0.125/0.5 dropped
    ids, p, _ = Vf.transform(x, [], Sampling(temperature=0.5))
    assert np.allclose(p, np.array([16, 4, 1, 1]) / 22, atol=1e-6)  # squared probabilities
    ids, p, _ = Vf.transform(x, [], Sampling(temperature=1.0, top_k=3))
    assert ids.tolist() == [0, 1, 2] and np.allclose(p, [4 / 7, 2 / 7, 1 / 7], atol=1e-7)
    # ties at the top-k cut go to the lower id: 2 and 3 tie, k = 3 keeps 2
    ids, _, _ = Vf.transform(x[[0, 1, 3, 2]], [], Sampling(temperature=1.0, top_k=3))
    assert ids.tolist() == [0, 1, 2]


def test_penalty_order_before_topk():
    # token 0 is the largest but penalised below token 1 -> top_k=1 picks 1
    x = np.array([3.0, 2.0, 0.0], np.float32)
    ids, _, _ = Vf.transform(x, [0], Sampling(temperature=1.0, repeat_penalty=2.0, top_k=1))
    assert ids.tolist() == [1]


def test_invcdf_hand_example():
    ids = np.array([2, 5, 9])
    w = np.array([0.2, 0.3, 0.5])
    assert Vf.invcdf(ids, w, 0.1)[0] == 2
    assert Vf.invcdf(ids, w, 0.25)[0] == 5
    assert Vf.invcdf(ids, w, 0.6)[0] == 9
    assert Vf.invcdf(ids, np.array([0.0, 0.3, 0.0]), 0.99)[0] == 5     # zero weights never chosen
    assert Vf.invcdf(ids, w * 10, 0.25)[0] == 5                       # unnormalised weights


def test_greedy_verify_hand_example():
    v = 12
    rows = np.zeros((3, v), np.float32)
    rows[0, 5] = rows[1, 7] = rows[2, 9] = 1.0
    ring = np.zeros(4, np.int32)
    st = np.array([0, 0], np.int32)
    r = Vf.verify(Sampling(), rows, None, [5, 8], ring, st)
    assert (r["k"], r["tokens"]) == (1, [5, 7])
    r = Vf.verify(Sampling(), rows, None, [5, 7], ring, st)
    assert (r["k"], r["tokens"]) == (2, [5, 7, 9])
    assert r["ring"].tolist()[:3] == [5, 7, 9] and r["state"].tolist() == [3, 3]
    r = Vf.verify(Sampling(), rows, None, [4, 7], ring, st)
    assert (r["k"], r["tokens"]) == (0, [5])


def test_greedy_penalty_window_includes_drafts():
    # row 1's argmax is token 3, but 3 was drafted at row 0 -> penalised below token 4
    rows = np.array([[0, 0, 0, 2, 0, 0], [0, 0, 0, 2.0, 1.9, 0], [1, 0, 0, 0, 0, 0]], np.float32)
    r = Vf.verify(Sampling(repeat_penalty=1.5, window=8), rows, None, [3, 4],
                  np.zeros(8, np.int32), np.array([0, 0], np.int32))
    assert (r["k"], r["tokens"]) == (2, [3, 4, 0])


def test_window_shorter_history_penalises_all():
    """A ring holding fewer tokens than the window penalises every token it
    holds (hand examples with 3 and 6 tokens in a window of 8)."""
    ring = np.array([4, 2, 0, 0, 0, 0, 0, 0], np.int32)
    st = np.array([2, 2], np.int32)                          # holds 4, 2
    assert Vf.window_for_row(Vf.ring_tokens(ring, st), [7, 9], 1, 8) == [4, 2, 7]
    assert Vf.window_for_row([1, 2, 3, 4, 5], [6], 1, 4) == [3, 4, 5, 6]
    ring6 = np.array([4, 2, 5, 3, 6, 1, 0, 0], np.int32)
    st6 = np.array([6, 6], np.int32)                         # holds 4, 2, 5, 3, 6, 1 (oldest first)
    assert Vf.window_for_row(Vf.ring_tokens(ring6, st6), [], 0, 8) == [4, 2, 5, 3, 6, 1]
    # token 4 (oldest in the ring, value 2.0) is penalised to 1.0, so token 8 (1.5) wins
    x = np.ones((1, 10), np.float32)
    x[0, 4], x[0, 8] = 2.0, 1.5
    r = Vf.verify(Sampling(repeat_penalty=2.0, window=8), x, None, [], ring6, st6)
    assert r["tokens"] == [8]


def test_ring_wraps():
    ring, st = Vf.ring_push(np.zeros(3, np.int32), np.array([0, 0], np.int32), [1, 2, 3, 4, 5])
    assert Vf.ring_tokens(ring, st) == [3, 4, 5] and st.tolist() == [2, 3]


# ---------------------------------------------------------------- brute force
V, N, L = 4, 2, 3
SP = Sampling(temperature=1.3, repeat_penalty=1.2, top_k=3, top_p=0.9, min_p=0.05, window=3)


def ctx_row(kind, ctx):
    """Seeded logits for a context (the committed-plus-drafted tokens so far); the
    draft row is the target row plus noise, so drafts are often accepted."""
    base = np.random.default_rng([7] + [t + 1 for t in ctx]).standard_normal(V) * 1.5
    if kind == "q":
        base = base + 1.2 * np.random.default_rng([8] + [t + 1 for t in ctx]).standard_normal(V)
    return base.astype(np.float32)


def dist(kind, ctx, hist):
    win = Vf.window_for_row(hist, [], 0, SP.window)
    ids, p, _ = Vf.transform(ctx_row(kind, ctx), win, SP)
    out = np.zeros(V)
    out[ids] = p
    return out


def seq_prob_sequential(seq, ctx0, hist0):
    pr = 1.0
    ctx, hist = list(ctx0), list(hist0)
    for t in seq:
        pr *= dist("p", ctx, hist)[t]
        ctx.append(t)
        hist.append(t)
    return pr


def round_outcomes(ctx, hist):
    """All outcomes of one verify round with their exact probabilities, found by
    calling the oracle's verify at representative uniforms (midpoints of the
    intervals on which its decisions are constant)."""
    res = {}
    ring = np.array(hist[-SP.window:] + [0] * (SP.window - len(hist[-SP.window:])), np.int32)
    st = np.array([len(hist[-SP.window:]) % SP.window, len(hist[-SP.window:])], np.int32)
    for d in itertools.product(range(V), repeat=N):
        qs = [dist("q", ctx + list(d[:i]), hist + list(d[:i])) for i in range(N)]
        ps = [dist("p", ctx + list(d[:i]), hist + list(d[:i])) for i in range(N + 1)]
        pd = math.prod(qs[i][d[i]] for i in range(N))
        if pd == 0:
            continue
        rows = np.stack([ctx_row("p", ctx + list(d[:i])) for i in range(N + 1)])
        drows = np.stack([ctx_row("q", ctx + list(d[:i])) for i in range(N)])
        # enumerate the path: first rejection index r (N = none)
        for r in range(N + 1):
            w_path, us = pd, []
            for i in range(r):
                b = min(1.0, ps[i][d[i]] / qs[i][d[i]])
                w_path *= b
                us.append(b / 2)
            if r < N:
                b = min(1.0, ps[r][d[r]] / qs[r][d[r]])
                w_path *= (1 - b)
                us.append((1 + b) / 2)
                fin = np.maximum(ps[r] - qs[r], 0)
                if fin.sum() == 0:
                    fin = ps[r]
            else:
                fin = ps[N]
            if w_path == 0:
                continue
            us += [0.5] * (N - len(us))
            c = np.cumsum(fin / fin.sum())
            lo = 0.0
            for j in range(V):
                if c[j] - lo > 0:
                    u = np.array(us + [(lo + c[j]) / 2], np.float32)
                    out = Vf.verify(SP, rows, drows, list(d), ring, st, u)
                    key = tuple(out["tokens"])
                    res[key] = res.get(key, 0.0) + w_path * (c[j] - lo)
                lo = c[j]
    return res


def test_rejection_sampling_preserves_target_distribution():
    """Rounds of draft + verify, expanded exactly, give every length-L token
    sequence the probability sequential sampling from the transformed target gives
    it (the pages' claim that greedy and sampled MTP only change speed)."""
    ctx0, hist0 = [2], [1, 2]
    states = {(): 1.0}
    final = {}
    while states:
        nxt = {}
        for seq, pr in states.items():
            if len(seq) >= L:
                final[seq[:L]] = final.get(seq[:L], 0.0) + pr
                continue
            for toks, w in round_outcomes(ctx0 + list(seq), hist0 + list(seq)).items():
                key = seq + toks
                nxt[key] = nxt.get(key, 0.0) + pr * w
        states = nxt
    # every path kind occurs: full acceptance (k = N) and rejection at each position
    first = round_outcomes(ctx0, hist0)
    assert {len(t) for t in first} == set(range(1, N + 2))
    assert min(sum(w for t, w in first.items() if len(t) == n) for n in range(1, N + 2)) > 0.05
    total = 0.0
    for seq in itertools.product(range(V), repeat=L):
        want = seq_prob_sequential(seq, ctx0, hist0)
        got = final.get(seq, 0.0)
        assert abs(got - want) < 1e-12, (seq, got, want)
        total += got
    assert abs(total - 1.0) < 1e-9


def test_sampled_monte_carlo_first_token():
    """Seeded uniforms: the first committed token's frequency matches p_0 (chi^2)."""
    rng = np.random.default_rng(11)
    ctx, hist = [1], [1]
    p0 = dist("p", ctx, hist)
    ring = np.array([1, 0, 0], np.int32)
    st = np.array([1, 1], np.int32)
    counts = np.zeros(V)
    trials = 4000
    for t in range(trials):
        d = []
        for i in range(N):
            q = dist("q", ctx + d, hist + d)
            d.append(int(rng.choice(V, p=q)))
        rows = np.stack([ctx_row("p", ctx + d[:i]) for i in range(N + 1)])
        drows = np.stack([ctx_row("q", ctx + d[:i]) for i in range(N)])
        out = Vf.verify(SP, rows, drows, d, ring, st, rng.random(N + 1).astype(np.float32))
        counts[out["tokens"][0]] += 1
    m = p0 > 0
    chi2 = np.sum((counts[m] - trials * p0[m]) ** 2 / (trials * p0[m]))
    assert chi2 < 25.0                                   # df <= 3; p ~ 1e-5
    assert np.all(counts[~m] == 0)


def test_sample_helper_matches_bonus_path():
    rows = np.random.default_rng(3).standard_normal((1, 30)).astype(np.float32)
    ring, st = np.array([4, 5, 6], np.int32), np.array([0, 3], np.int32)
    for u in (0.01, 0.3, 0.77, 0.999):
        sp = Sampling(temperature=0.7, repeat_penalty=1.1, top_k=10, top_p=0.9, window=3)
        a = Vf.sample(sp, rows[0], ring, st, u)
        b = Vf.verify(sp, rows, np.zeros((0, 30), np.float32), [], ring, st,
                      np.array([u], np.float32))["tokens"][0]
        assert a == b
