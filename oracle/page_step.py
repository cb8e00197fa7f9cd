"""Second, independent oracle: the blog engine's own step semantics (tests only).

Test infrastructure; only the tests use it. It re-expresses, from the prose and
the behaviour of the reference engine in the LongFlow Guide
(§End-to-End Implementation: Building a LongFlow Engine), what one call of
that engine does, in float64 NumPy written for this project:

  * the buffer holds `budget` slots per head; while not full, the incoming
    token takes the next free slot;
  * once full, the incoming token takes the slot that the PREVIOUS call chose
    as its victim (the engine falls back to the last slot when no victim has
    been chosen yet);
  * the call then attends over every occupied slot (the incoming token
    included), per head, with scale 1/sqrt(d);
  * every occupied slot is scored by the l1 norm of its explicit contribution
    tensor alpha_{h,i} * v_{h,i,:}, summed over heads and features;
  * the first `sink_size` slots and the slot just written are shielded; the
    slot with the smallest remaining score (first one on ties) becomes the
    victim for the NEXT call.

The tests run it with budget B+1 against longflow_oracle with budget B and
check that both evict the same token positions in the same order: each step
of either attends the same token set and shields the same newest token.
"""
from __future__ import annotations

import numpy as np


class DeferredEvictionEngine:
    """Multi-head engine with a deferred victim; all heads share one slot choice."""

    def __init__(self, num_heads: int, head_dim: int, budget: int, sink_size: int = 0):
        self.h, self.d, self.budget, self.sink = num_heads, head_dim, budget, sink_size
        self.keys = np.zeros((num_heads, budget, head_dim))
        self.vals = np.zeros((num_heads, budget, head_dim))
        self.used = 0
        self.victim = None
        self.token_at = np.full(budget, -1, dtype=np.int64)   # token id held by each slot

    def load(self, keys: np.ndarray, vals: np.ndarray, token_ids) -> None:
        """Place m tokens in slots 0..m-1 without attending (a prompt)."""
        m = keys.shape[1]
        self.keys[:, :m] = keys
        self.vals[:, :m] = vals
        self.token_at[:m] = token_ids
        self.used = m

    def _target_slot(self) -> int:
        if self.used < self.budget:
            slot = self.used
            self.used += 1
            return slot
        return self.budget - 1 if self.victim is None else self.victim

    def advance(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, token_id: int):
        """One call: q, k, v are [heads][d]. Returns (out [heads][d], replaced token id)."""
        slot = self._target_slot()
        replaced = int(self.token_at[slot])
        self.keys[:, slot] = k
        self.vals[:, slot] = v
        self.token_at[slot] = token_id
        live_k = self.keys[:, :self.used]            # [H][m][d]
        live_v = self.vals[:, :self.used]
        tau = 1.0 / np.sqrt(self.d)
        logits = np.einsum("hd,hmd->hm", q, live_k) * tau
        w = np.exp(logits - logits.max(axis=1, keepdims=True))
        probs = w / w.sum(axis=1, keepdims=True)
        contrib = probs[:, :, None] * live_v          # c_{h,i,:}
        out = contrib.sum(axis=1)
        slot_score = np.abs(contrib).sum(axis=(0, 2))
        slot_score[:self.sink] = np.inf
        slot_score[slot] = np.inf
        self.victim = int(np.argmin(slot_score))
        return out, replaced
