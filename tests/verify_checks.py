"""Validity of a sampled-verification outcome in a boundary round (host only).

A round whose oracle decision margin (top-p crossing, accept test, inverse-CDF
step) lies below the band may legitimately end differently in fp32 than in the
oracle's fp64.  ``check_boundary`` accepts an outcome only if it is one of the
correct ones: every accept decision consistent with p and q (or inside the
band), the final token in the support of normalise(max(0, p_k - q_k)) (p_k when
that is empty; p_N for the bonus), where a top-p cut inside the band admits the
cut one token either side, and the history ring equal to the push of the
outcome's own tokens."""
import dataclasses

import numpy as np

from oracle import verify as OV


def admissible(sp_o, row, win, band):
    """The transforms of one row an fp32 computation may legitimately produce:
    the oracle's, and where its top-p cut lies within the band of a cumulative
    sum, the cuts one token earlier and later."""
    ids, p, info = OV.transform(row, win, sp_o)
    out = [(ids, p)]
    if info["top_p_margin"] < band:
        for tp in (sp_o.top_p - 2 * band, sp_o.top_p + 2 * band):
            if 0.0 < tp < 1.0:
                out.append(OV.transform(row, win, dataclasses.replace(sp_o, top_p=tp))[:2])
    return out


def check_boundary(sp_o, rows, drows, d, ring, st, u, got, band):
    """Full validity of a boundary round's GPU outcome (see the module text)."""
    n = len(d)
    k = got["k"]
    assert 0 <= k <= n and got["count"] == k + 1 and got["tokens"][:k] == [int(t) for t in d[:k]]
    history = OV.ring_tokens(ring, st)
    u = np.asarray(u, np.float64)
    for i in range(min(k + 1, n)):           # every accept test the GPU ran
        win = OV.window_for_row(history, d, i, sp_o.window)
        accepted = i < k
        ok = False
        for pi, pp in admissible(sp_o, rows[i], win, band):
            for qi, qp in admissible(sp_o, drows[i], win, band):
                pd, qd = OV.prob_of(pi, pp, int(d[i])), OV.prob_of(qi, qp, int(d[i]))
                lhs = u[i] * qd
                if (lhs < pd) == accepted or abs(pd - lhs) / max(pd, lhs, 1e-300) < band:
                    ok = True
        assert ok, ("accept decision", i, accepted)
    win = OV.window_for_row(history, d, k, sp_o.window)
    support = set()
    for pi, pp in admissible(sp_o, rows[k], win, band):
        if k == n:
            support |= {int(t) for t, w in zip(pi, pp) if w > 0}
            continue
        for qi, qp in admissible(sp_o, drows[k], win, band):
            ids = np.union1d(pi, qi)
            r = [max(0.0, OV.prob_of(pi, pp, t) - OV.prob_of(qi, qp, t)) for t in ids]
            if sum(r) > 0.0:
                support |= {int(t) for t, w in zip(ids, r) if w > 0}
            else:
                support |= {int(t) for t, w in zip(pi, pp) if w > 0}
    assert int(got["tokens"][k]) in support, ("final token outside the support", k, got["tokens"][k])
    want_ring, want_state = OV.ring_push(ring, st, got["tokens"])
    assert np.array_equal(got["ring"], want_ring) and np.array_equal(got["state"], want_state)


