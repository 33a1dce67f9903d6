"""Oracle: the MTP round driver.  TEST INFRASTRUCTURE ONLY.

One round (greedy drafting):
  1. flush the pending completed pairs in LAST mode and record the round base;
     its last row yields d_0 (argmax) and g_0;
  2. N - 1 chained steps, each feeding (d_{i-1}, g_{i-1}) at the next slot;
  3. one target forward over [current, d_0 .. d_{N-1}] (N + 1 rows, supplied by
     a callback standing in for the target model);
  4. verify -> k accepted drafts and k + 1 committed tokens;
  5. draft-KV rollback and re-pairing.  The pair at slot C + j is
     (committed token j, target hidden row j), j = 0..k.
     Policy A rolls back to the round base and leaves all k + 1 pairs pending;
     policy B keeps the chained entries of accepted drafts, base + min(k, N - 1),
     and leaves pairs j = min(k, N - 1)..k pending.

Sources: "Ollama qwen3_5 MTP loader and SelfDraft path", Facts "MTP drafting"
(slot S pairs the token at S + 1 with the target hidden at S, a pair completes
when the next token arrives, flushes of up to 256), Facts "Verification" (one
target forward over the current token plus drafts, one host sync per round) and
the Ollama commit log (the committed run is reported to the drafter, which pairs
and flushes; greedy as the point-mass case of sampling).  Block size is the round
budget including the bonus token, so N = block_size - 1 drafts and N + 1
verified rows ("feat(inference): support the qwen3_5_mtp drafter ...", section
"Upstream contract to port").

Invariant after every round: kv.len + len(pending) == len(committed) - 1.
"""
from __future__ import annotations

import numpy as np

from .head import LAST, KV_ONLY
from .kvcache import ROUND_BASE
from .verify import Sampling, verify, penalize, ring_tokens, ring_push, window_for_row

GREEDY = Sampling()


class RoundState:
    def __init__(self, head, kv, pending, committed, ring=None, ring_state=None, window=64):
        self.head, self.kv = head, kv
        self.pending = list(pending)          # [(token, hidden)]
        self.committed = list(committed)
        if ring is None:
            ring = np.zeros(window, dtype=np.int32)
            ring_state = np.array([0, 0], dtype=np.int32)
        self.ring, self.ring_state = np.array(ring, dtype=np.int32), np.array(ring_state, dtype=np.int32)

    def invariant(self) -> bool:
        return self.kv.len + len(self.pending) == len(self.committed) - 1


def run_round(st: RoundState, n_draft: int, target_fn, sp: Sampling = GREEDY,
              policy: str = "A", uniforms=None, draft_rows_fn=None, forced_drafts=None):
    """Run one round in place.  ``target_fn(tokens_in, start_pos)`` returns
    (logits [N + 1, V] fp32, hiddens [N + 1, H]) for tokens_in = [current] + drafts
    processed at positions start_pos + j.  Returns a dict with the drafts, k, the
    committed tokens and each draft step's logits and hidden output g.

    ``forced_drafts`` (comparisons only) replaces each step's argmax by the given
    token when the chain continues, so a run can follow another implementation
    through a near tie; the returned logits are still this oracle's own."""
    head, kv = st.head, st.kv
    toks = [t for t, _ in st.pending]
    hids = [h for _, h in st.pending]
    out = head.flush(kv, toks, hids, LAST, set_round_base=True)

    def pick(i, o):
        return int(forced_drafts[i]) if forced_drafts is not None else o["argmax"]
    drafts = [pick(0, out)]
    draft_logits = [out["logits"]]
    g = out["g"][-1]
    draft_g = [g]
    for i in range(1, n_draft):
        o = head.step(kv, drafts[-1], g)
        drafts.append(pick(i, o))
        draft_logits.append(o["logits"])
        g = o["g"][-1]
        draft_g.append(g)
    c = len(st.committed) - 1                    # position of the current token
    rows, hid_rows = target_fn([st.committed[-1]] + drafts, c)
    draft_rows = draft_rows_fn(drafts) if draft_rows_fn is not None else None
    res = verify(sp, rows, draft_rows, drafts, st.ring, st.ring_state, uniforms)
    k, committed = res["k"], res["tokens"]
    st.ring, st.ring_state = res["ring"], res["state"]
    if policy == "A":
        kv.rollback(ROUND_BASE)
        j0 = 0
    elif policy == "B":
        kv.rollback(ROUND_BASE, n_accepted=k, n_draft=n_draft)
        j0 = min(k, n_draft - 1)
    else:
        raise ValueError(policy)
    st.pending = [(committed[j], hid_rows[j]) for j in range(j0, k + 1)]
    st.committed.extend(committed)
    return {"drafts": drafts, "k": k, "tokens": committed, "draft_logits": draft_logits, "draft_g": draft_g}


def classic_greedy(target_fn, committed, n_new: int, sp: Sampling = GREEDY, ring=None, ring_state=None):
    """Plain sequential greedy decoding of the target alone: each new token is the
    argmax of the (penalised) row for the previous token."""
    out = list(committed)
    if ring is None:
        ring = np.zeros(sp.window, dtype=np.int32)
        ring_state = np.array([0, 0], dtype=np.int32)
    for _ in range(n_new):
        rows, _ = target_fn([out[-1]], len(out) - 1)
        win = window_for_row(ring_tokens(ring, ring_state), [], 0, sp.window)
        row = penalize(rows[0], win, sp.repeat_penalty) if sp.repeat_penalty != 1.0 else rows[0]
        t = int(np.argmax(row))
        out.append(t)
        ring, ring_state = ring_push(ring, ring_state, [t])
    return out


def pairs_from_stream(committed, hidden_fn, start: int, stop: int):
    """Pairs (t_{S+1}, h_S) for slots S in [start, stop), with h_S = hidden_fn(S)."""
    return [(committed[s + 1], hidden_fn(s)) for s in range(start, stop)]


def rebuild_kv(head, kv_template, pairs, start: int):
    """A fresh KV equal to ``kv_template`` on [0, start) with ``pairs`` flushed
    from slot ``start`` in KV_ONLY mode."""
    kv = kv_template.copy()
    kv.len = start
    kv.err = 0
    head.flush(kv, [t for t, _ in pairs], [h for _, h in pairs], KV_ONLY)
    return kv
