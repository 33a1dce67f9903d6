"""Oracle: the draft KV cache with its append and rollback.  TEST INFRASTRUCTURE ONLY.

The draft head keeps its own K/V cache, separate from the target's; only the
offset is shared so that slot S sits at position S ("feat(inference): support the
qwen3_5_mtp drafter ...", section "Upstream contract to port", on the separate
per-layer caches).  A rejected suffix is trimmed by moving the length back
(same page, the #1174 comment on trimming attention KV by the rejected count);
trimming never touches the bytes of the kept prefix.

Two rollback targets are supported.  Policy A ("Ollama qwen3_5 MTP loader and
SelfDraft path", Facts "MTP drafting" and the commit that makes the committed
stream the drafter's maintenance mechanism): every chained entry is provisional;
roll back to the round base and re-flush the completed pairs.  Policy B: keep the
chained entries whose draft token was accepted, base + min(k, N - 1), and trim
the rest.

Device-side errors are sticky: once ``err`` is non-zero every later append and
rollback is a no-op.
"""
from __future__ import annotations

import numpy as np

ROUND_BASE = -1
ERR_NONE, ERR_CAPACITY, ERR_ROLLBACK, ERR_COUNT = 0, 1, 2, 3


class DraftKV:
    def __init__(self, n_kv_heads, capacity, head_dim, K=None, V=None, length=0):
        self.K = np.zeros((n_kv_heads, capacity, head_dim), dtype=np.float64)
        self.V = np.zeros_like(self.K)
        if K is not None:
            self.K[...] = np.asarray(K, dtype=np.float64)
            self.V[...] = np.asarray(V, dtype=np.float64)
        self.capacity = capacity
        self.len = int(length)
        self.base = int(length)
        self.err = ERR_NONE

    def can_append(self, n: int) -> bool:
        if self.err:
            return False
        if self.len + n > self.capacity:
            self.err = ERR_CAPACITY
            return False
        return True

    def write(self, pos: int, k, v):
        self.K[:, pos] = k
        self.V[:, pos] = v

    def rollback(self, to_len: int = ROUND_BASE, n_accepted=None, n_draft: int = 0):
        """Set the length to ``to_len`` (>= 0), or with ROUND_BASE to the round
        base (policy A) or, when ``n_accepted`` is given, to
        base + min(n_accepted, n_draft - 1) (policy B).  A target beyond the
        current length is a device-side error and changes nothing."""
        if self.err:
            return
        if to_len == ROUND_BASE:
            to = self.base
            if n_accepted is not None:
                to = self.base + min(int(n_accepted), max(int(n_draft) - 1, 0))
        else:
            to = int(to_len)
        if to < 0 or to > self.len:
            self.err = ERR_ROLLBACK
            return
        self.len = to

    def copy(self) -> "DraftKV":
        c = DraftKV(self.K.shape[0], self.capacity, self.K.shape[2], self.K, self.V, self.len)
        c.base, c.err = self.base, self.err
        return c
