"""Oracle: speculative verification of drafted tokens against the target rows.
TEST INFRASTRUCTURE ONLY.

The round verifies N drafted tokens with one target forward over the current
token plus the drafts, i.e. N + 1 target logits rows ("Ollama qwen3_5 MTP loader
and SelfDraft path", Facts "Verification" and the commit that runs one target
forward per MTP decode step).  Verification is rejection sampling in the
Leviathan/Chen form (the Ollama commit log's DFlash change names it), and it
honours temperature, repetition penalty and top-k / top-p / min-p.  At
temperature 0 the sampler is a point mass, so acceptance reduces to "the draft
equals the argmax" (the commit that collapses the greedy, sampled and serial
paths into one).

Readings where the pages only list the features (no order, no formula):
  * sampler order: penalty, then temperature, then top-k, then softmax over the
    survivors, then top-p, then min-p, then renormalise;
  * the penalty applies once per distinct token of the window: a positive logit
    is divided by the penalty, a non-positive one multiplied; the window of
    target row i (and draft row i) is the last ``window`` tokens of the history
    followed by d_0..d_{i-1};
  * ordering everywhere is by value descending, then token id ascending;
  * top-p keeps the shortest sorted prefix whose cumulative mass reaches top_p
    (top_p >= 1 keeps all); min-p keeps tokens whose logit is within ln(min_p)
    of the maximum (min_p = 0 keeps all);
  * accept d_i iff u_i * q_i(d_i) < p_i(d_i); at the first rejection sample from
    normalise(max(0, p_i - q_i)) (p_i itself if that is all zero) with u_N; if
    every draft is accepted, sample the bonus token from p_N with u_N;
  * sampling by inverse CDF walks the support in ascending token id and returns
    the first id whose running sum exceeds u * total;
  * greedy (temperature 0) uses the penalised row's argmax (lowest id on ties);
  * the k + 1 committed tokens are pushed into the history ring.

Penalty, temperature, top-k and min-p decide which tokens survive; they are
computed in fp32 (IEEE division and subtraction, ln(min_p) rounded once from
fp64), the precision the kernel decides them in, so the surviving sets are
identical on both sides.  Probabilities and sums are fp64.  Every other decision
(top-p crossing, accept test, inverse-CDF step) records its margin so callers can
tell a real mismatch from an fp32-vs-fp64 boundary case.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Sampling:
    temperature: float = 0.0
    repeat_penalty: float = 1.0
    top_k: int = 0
    top_p: float = 1.0
    min_p: float = 0.0
    window: int = 64


# --------------------------------------------------------------------------
# history ring
# --------------------------------------------------------------------------
def ring_tokens(ring, state):
    """Tokens in the ring, oldest first; ``state`` = (head, count) with head the
    next write slot."""
    w = len(ring)
    head, count = int(state[0]), int(state[1])
    start = (head - count) % w if w else 0
    return [int(ring[(start + i) % w]) for i in range(count)]


def ring_push(ring, state, tokens):
    ring = np.array(ring, dtype=np.int32, copy=True)
    head, count = int(state[0]), int(state[1])
    w = len(ring)
    for t in tokens:
        if w == 0:
            break
        ring[head] = t
        head = (head + 1) % w
        count = min(count + 1, w)
    return ring, np.array([head, count], dtype=np.int32)


def window_for_row(history, drafts, i, window):
    """The last ``window`` tokens of history ++ d_0..d_{i-1} (all of them when
    there are fewer)."""
    seq = list(history) + [int(t) for t in drafts[:i]]
    return seq[max(0, len(seq) - window):] if window > 0 else []


# --------------------------------------------------------------------------
# the transform
# --------------------------------------------------------------------------
def penalize(x, window, penalty):
    """Repetition penalty on fp32 logits, once per distinct window token."""
    y = np.array(x, dtype=np.float32, copy=True)
    pen = np.float32(penalty)
    for t in sorted(set(int(w) for w in window)):
        v = y[t]
        y[t] = v / pen if v > 0 else v * pen
    return y


def transform(x, window, sp: Sampling):
    """Transformed distribution of one logits row.

    Returns (ids ascending int64, probabilities fp64, info) where info holds
    'top_p_margin' (distance of top_p from the nearest cumulative sum that
    decided the cut, inf when unused)."""
    y = penalize(x, window, sp.repeat_penalty) if sp.repeat_penalty != 1.0 else \
        np.array(x, dtype=np.float32, copy=True)
    y = (y / np.float32(sp.temperature)).astype(np.float32)
    v = y.shape[0]
    order = np.lexsort((np.arange(v), -y))          # value desc, id asc
    k = sp.top_k if 0 < sp.top_k < v else v
    sel = order[:k]
    ymax = y[sel[0]]
    p = np.exp(y[sel].astype(np.float64) - float(ymax))
    p /= p.sum()
    keep = k
    info = {"top_p_margin": math.inf}
    if sp.top_p < 1.0:
        c = np.cumsum(p)
        idx = int(np.searchsorted(c, sp.top_p, side="left"))
        idx = min(idx, k - 1)
        keep = idx + 1
        m = abs(c[idx] - sp.top_p)
        if idx > 0:
            m = min(m, abs(sp.top_p - c[idx - 1]))
        info["top_p_margin"] = m
    if sp.min_p > 0.0:
        thr = np.float32(math.log(sp.min_p))
        diff = (y[sel[:keep]] - ymax).astype(np.float32)
        keep = min(keep, int(np.count_nonzero(diff >= thr)))
    kept = sel[:keep]
    w = np.exp(y[kept].astype(np.float64) - float(ymax))
    w /= w.sum()
    o = np.argsort(kept, kind="stable")
    return kept[o].astype(np.int64), w[o], info


def prob_of(ids, probs, token):
    j = np.searchsorted(ids, token)
    return float(probs[j]) if j < len(ids) and ids[j] == token else 0.0


def invcdf(ids, weights, u):
    """First id (ascending) whose running weight sum exceeds u * total; the last
    positive-weight id if none does.  Returns (token, margin) with the margin
    relative to the total."""
    w = np.asarray(weights, dtype=np.float64)
    tot = w.sum()
    c = np.cumsum(w)
    t = float(u) * tot
    j = int(np.searchsorted(c, t, side="right"))
    if j >= len(c):
        j = int(np.nonzero(w > 0)[0][-1])
    lo = c[j - 1] if j > 0 else 0.0
    margin = min(c[j] - t, t - lo) / tot if tot > 0 else 0.0
    return int(ids[j]), margin


# --------------------------------------------------------------------------
# verification
# --------------------------------------------------------------------------
def verify(sp: Sampling, target_rows, draft_rows, drafts, ring, ring_state, uniforms=None):
    """Verify N = len(drafts) drafts against N + 1 target rows.

    Returns dict(k=accepted count, tokens=[k + 1 committed ids], ring, state,
    margin=smallest decision margin on the path taken (inf for greedy))."""
    n = len(drafts)
    target_rows = np.asarray(target_rows, dtype=np.float32)
    history = ring_tokens(ring, ring_state)
    margin = math.inf
    if sp.temperature == 0.0:
        toks = []
        k = n
        for i in range(n + 1):
            win = window_for_row(history, drafts, i, sp.window)
            row = penalize(target_rows[i], win, sp.repeat_penalty) \
                if sp.repeat_penalty != 1.0 else target_rows[i]
            a = int(np.argmax(row))
            if i < n and int(drafts[i]) == a:
                toks.append(a)
                continue
            toks.append(a)
            k = i
            break
    else:
        draft_rows = np.asarray(draft_rows, dtype=np.float32)
        u = np.asarray(uniforms, dtype=np.float64)
        toks, k = None, n
        for i in range(n):
            win = window_for_row(history, drafts, i, sp.window)
            pid, pp, pinfo = transform(target_rows[i], win, sp)
            qid, qp, qinfo = transform(draft_rows[i], win, sp)
            margin = min(margin, pinfo["top_p_margin"], qinfo["top_p_margin"])
            d = int(drafts[i])
            pd, qd = prob_of(pid, pp, d), prob_of(qid, qp, d)
            lhs = u[i] * qd
            margin = min(margin, abs(pd - lhs) / max(pd, lhs, 1e-300))
            if lhs < pd:
                continue
            ids = np.union1d(pid, qid)
            r = np.array([max(0.0, prob_of(pid, pp, t) - prob_of(qid, qp, t)) for t in ids])
            if r.sum() > 0.0:
                tok, m = invcdf(ids, r, u[n])
            else:
                tok, m = invcdf(pid, pp, u[n])
            margin = min(margin, m)
            toks = [int(t) for t in drafts[:i]] + [tok]
            k = i
            break
        if toks is None:
            win = window_for_row(history, drafts, n, sp.window)
            pid, pp, pinfo = transform(target_rows[n], win, sp)
            tok, m = invcdf(pid, pp, u[n])
            margin = min(margin, pinfo["top_p_margin"], m)
            toks = [int(t) for t in drafts] + [tok]
    new_ring, new_state = ring_push(ring, ring_state, toks)
    return {"k": k, "tokens": toks, "ring": new_ring, "state": new_state, "margin": margin}


def sample(sp: Sampling, row, ring, ring_state, u, prefix=()):
    """Draw one token from a single row with the same transform (the window is the
    history followed by ``prefix``); the ring is not touched.  This is how a
    drafter that samples would draw d_i from its own row i."""
    history = ring_tokens(ring, ring_state)
    win = window_for_row(history, list(prefix), len(prefix), sp.window)
    if sp.temperature == 0.0:
        r = penalize(row, win, sp.repeat_penalty) if sp.repeat_penalty != 1.0 else row
        return int(np.argmax(r))
    ids, p, _ = transform(row, win, sp)
    return invcdf(ids, p, u)[0]
