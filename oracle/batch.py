"""Oracle: B > 1 independent sessions with ragged acceptance.  TEST
INFRASTRUCTURE ONLY.

A batched round is, session by session, the single-session round of
``rounds.run_round``: every session has its own draft KV (its own length and
round base), its own pending pairs, history ring and target rows, and accepts
its own number of drafts; nothing is shared between sessions but the head's
weights.  So the batch oracle is a loop over the sessions.

Sources: "feat(inference): support the qwen3_5_mtp drafter ...", section
"Upstream contract to port" (the drafter advertises ragged batch acceptance and
does not require uniform acceptance), sections "Implementation plan" and
"Acceptance criteria" (B > 1 lands behind a passing ragged-acceptance test, or
is rejected with a named error), and the #1174 comment (each row is trimmed by
its own accepted count; a shared-offset batch cache zeroes each row's tail).
Reading: with one length per session no slot past a session's length is ever
read, so the per-row tail zeroing of a shared-offset cache has no counterpart
here; the committed streams and every session's KV prefix are what must match.
"""
from __future__ import annotations

from .rounds import GREEDY, run_round


def run_batch_round(states, n_draft, target_fns, sp=GREEDY, policy="A", uniforms=None, draft_rows_fns=None,
                    forced_drafts=None):
    """One round of every session: ``states`` [B] RoundState, ``target_fns`` [B]
    target callbacks (as for run_round), optional per-session uniforms, draft
    rows and forced drafts.  Returns the list of per-session round results."""
    out = []
    for b, st in enumerate(states):
        out.append(run_round(st, n_draft, target_fns[b], sp=sp, policy=policy,
                             uniforms=None if uniforms is None else uniforms[b],
                             draft_rows_fn=None if draft_rows_fns is None else draft_rows_fns[b],
                             forced_drafts=None if forced_drafts is None else forced_drafts[b]))
    return out
