"""Float64 CPU oracle of one LongFlow decode step (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module; the product path never does.

What it computes, for one pair (sequence b, KV head h) holding n cached tokens
in a static buffer of B slots, a query group q_0..q_{G-1} (the G query heads
that share KV head h) and the new token (k_new, v_new):

  1. The attended set A is the n cached tokens plus the new token (the new
     token attends to itself, as in the reference engine of the LongFlow Guide,
     §End-to-End Implementation, which stores the token before attending).
  2. s_{g,i} = tau * <q_g, k_i>, tau = 1/sqrt(d) unless overridden.
  3. alpha_{g,i} = exp(s_{g,i}) / sum_{j in A} exp(s_{g,j}).
     (LongFlow Guide, §Mathematical Derivation of the LongFlow Score, the
     alpha equation.)
  4. out_g = sum_{i in A} alpha_{g,i} v_i  (same section, the o_t equation).
  5. Below the budget (n < B) the token is appended at slot n and nothing is
     evicted (LongFlow Guide, §Static Memory Pre-Allocation and In-Place
     Eviction, item 1 "Initial Fill").
  6. At the budget (n == B) every cached slot i in [sink_size, B) gets
        score_i = ||v_i||_1 * sum_g alpha_{g,i}
     which is the l1 norm of token i's contribution vectors c_{g,i} =
     alpha_{g,i} v_i summed over the group (same Guide section, the c_{t,i}
     and Score equations; gist.science summary §2.1, LongFlowScore =
     alpha * ||v||_1). The new token is never a candidate. The slot with the
     smallest score, lowest index on ties, receives k_new, v_new and
     ||v_new||_1 (Guide, §Static Memory..., items 2-3).

Readings taken where the pages are silent or ambiguous (each listed in the
design notes): the score is summed over the G query heads of one KV head and
uses each head's own normalised alpha (the blog's code sums over all heads of
a sequence); the ordering is score -> argmin -> write within one step (the
blog defers the write to the next step; run with one more slot, that order
evicts the same tokens, which the tests check against order="deferred");
sinks default to 0; ||v||_1 is taken over the stored values.

Variants (each a runtime option of the same step; the defaults above are the
main path):

  * norm="l2": the score uses ||v_i||_2 in place of ||v_i||_1, i.e. the l2
    norm of each head's contribution vector alpha_{g,i} v_i, summed over the
    group (Guide, §Mathematical Derivation: the score may take the l1 or the
    l2 norm of c_{t,i}).
  * order="deferred": the blog engine's own order (Guide, §End-to-End
    Implementation). Once the buffer is full the new token is first written
    into the slot chosen as victim by the PREVIOUS step (the last slot when
    no victim has been chosen yet); the step then attends over the occupied
    slots, new token included, and, if the buffer is full after the write,
    scores the cached slots (sinks and the slot just written shielded) and
    keeps the first argmin as the next victim.
  * scope="sequence" (LayerCache): one victim per sequence, from the sum over
    its KV heads of their group scores (the blog engine sums the contribution
    norm over all heads); every KV head of the sequence evicts the same slot.

All arithmetic is float64. Inputs must be finite.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

NEAR_TIE_REL = 1e-4
NEAR_TIE_ABS = 1e-30


def default_scale(head_dim: int) -> float:
    """tau = 1/sqrt(d) (Guide, §Mathematical Derivation, the alpha equation)."""
    return 1.0 / np.sqrt(float(head_dim))


def attention_logits(q: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """s_{g,i} = tau * q_g . k_i ; q [G][d], keys [m][d] -> [G][m]."""
    return scale * (np.asarray(q, np.float64) @ np.asarray(keys, np.float64).T)


def attention_weights(q: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """alpha_{g,i}: softmax of the logits over the attended tokens, per query head.

    The common factor exp(-max_i s_{g,i}) is taken out of numerator and
    denominator to keep exp() finite; the quotient is unchanged.
    """
    s = attention_logits(q, keys, scale)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def attention_output(alpha: np.ndarray, values: np.ndarray) -> np.ndarray:
    """o_g = sum_i alpha_{g,i} v_i ; alpha [G][m], values [m][d] -> [G][d]."""
    return alpha @ np.asarray(values, np.float64)


def l1_norms(values: np.ndarray) -> np.ndarray:
    """||v_i||_1 for each row."""
    return np.abs(np.asarray(values, np.float64)).sum(axis=-1)


def l2_norms(values: np.ndarray) -> np.ndarray:
    """||v_i||_2 for each row."""
    v = np.asarray(values, np.float64)
    return np.sqrt((v * v).sum(axis=-1))


def value_norms(values: np.ndarray, norm: str) -> np.ndarray:
    """The per-token sidecar: ||v_i||_1 or ||v_i||_2."""
    if norm == "l1":
        return l1_norms(values)
    if norm == "l2":
        return l2_norms(values)
    raise ValueError(f"unknown norm {norm!r}")


def longflow_scores(alpha: np.ndarray, vnorm: np.ndarray) -> np.ndarray:
    """score_i = ||v_i|| * sum_g alpha_{g,i}: the norm of each head's
    contribution vector alpha_{g,i} v_i (alpha >= 0), summed over the group;
    alpha [G][m], vnorm [m] -> [m]."""
    return np.asarray(vnorm, np.float64) * alpha.sum(axis=0)


def first_argmin(scores: np.ndarray) -> int:
    """Smallest index attaining the minimum (lowest slot wins ties)."""
    m = np.min(scores)
    return int(np.flatnonzero(scores == m)[0])


def near_tie_set(scores: np.ndarray):
    """(is_near_tie, legal slots) for a candidate score vector.

    Let s1 <= s2 be the two lowest finite candidates. The step is a near-tie
    iff s2 - s1 < 1e-4 * s2, or s2 < 1e-30. Then any slot i with
    score_i - s1 < 1e-4 * s2 (or score_i <= 1e-30 in the underflow case) is a
    legal choice; otherwise only the first argmin is.
    """
    finite = np.flatnonzero(np.isfinite(scores))
    best = first_argmin(scores)
    if finite.size < 2:
        return False, [best]
    vals = np.sort(scores[finite])
    s1, s2 = float(vals[0]), float(vals[1])
    tie = (s2 - s1) < NEAR_TIE_REL * s2 or s2 < NEAR_TIE_ABS
    if not tie:
        return False, [best]
    thresh = max(NEAR_TIE_REL * s2, 0.0)
    legal = [int(i) for i in finite if scores[i] - s1 < thresh
             or scores[i] <= NEAR_TIE_ABS]
    if best not in legal:
        legal.append(best)
    return True, sorted(legal)


@dataclass
class StepResult:
    out: np.ndarray                 # [G][d] float64
    alpha: np.ndarray               # same-step: [G][n+1], last column = new token;
                                    # deferred: [G][n_after], column = slot (new token at `slot`)
    scores: Optional[np.ndarray]    # [B] float64, +inf for non-candidates; None if not scored
    evicted: int                    # slot whose token is replaced this step, -1 when appended
    slot: int                       # slot the new token is written to
    near_tie: bool                  # about the choice made this step (same-step: `evicted`,
    legal: list                     # deferred: `next_victim`), with its legal slots
    next_victim: int = -1           # deferred: victim for the next step, -1 = none


ORDERS = ("same_step", "deferred")
NORMS = ("l1", "l2")


class PairCache:
    """One (layer, sequence, KV head) region of the static cache, in float64.

    evict=True  -> LongFlow: `budget` slots, eviction once full.
    evict=False -> full-KV baseline: capacity `budget`, never evicts; a step
                   that would exceed capacity is an error.
    norm, order -> the variants described in the module docstring.
    """

    def __init__(self, budget: int, head_dim: int, sink_size: int = 0,
                 evict: bool = True, scale: Optional[float] = None,
                 norm: str = "l1", order: str = "same_step"):
        if budget <= 0 or head_dim <= 0:
            raise ValueError("budget and head_dim must be positive")
        if not 0 <= sink_size < budget:
            raise ValueError("sink_size must be in [0, budget)")
        if norm not in NORMS or order not in ORDERS:
            raise ValueError("unknown norm or order")
        self.budget = budget
        self.head_dim = head_dim
        self.sink_size = sink_size
        self.evict = evict
        self.norm = norm
        self.order = order
        self.scale = default_scale(head_dim) if scale is None else float(scale)
        self.K = np.zeros((budget, head_dim))
        self.V = np.zeros((budget, head_dim))
        self.vnorm = np.zeros(budget)
        self.n = 0
        self.victim = -1

    def copy(self) -> "PairCache":
        c = PairCache(self.budget, self.head_dim, self.sink_size, self.evict, self.scale,
                      self.norm, self.order)
        c.K, c.V, c.vnorm = self.K.copy(), self.V.copy(), self.vnorm.copy()
        c.n, c.victim = self.n, self.victim
        return c

    def prefill(self, k_rows: np.ndarray, v_rows: np.ndarray) -> None:
        """Tokens go to slots 0..m-1 in order; m > budget is an error."""
        k_rows = np.asarray(k_rows, np.float64)
        v_rows = np.asarray(v_rows, np.float64)
        m = k_rows.shape[0]
        if m > self.budget:
            raise ValueError("prefill longer than the budget")
        self.K[:m] = k_rows
        self.V[:m] = v_rows
        self.vnorm[:m] = value_norms(v_rows, self.norm)
        self.K[m:] = 0.0
        self.V[m:] = 0.0
        self.vnorm[m:] = 0.0
        self.n = m
        self.victim = -1

    def reset(self) -> None:
        """Recycle the region for a new sequence: no token, no victim."""
        self.n = 0
        self.victim = -1

    def attend(self, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray) -> StepResult:
        """One step without mutating the cache."""
        q = np.asarray(q, np.float64)
        k_new = np.asarray(k_new, np.float64)
        v_new = np.asarray(v_new, np.float64)
        for arr in (q, k_new, v_new):
            if not np.all(np.isfinite(arr)):
                raise ValueError("inputs must be finite")
        if self.evict and self.order == "deferred":
            return self._attend_deferred(q, k_new, v_new)
        n = self.n
        keys = np.vstack([self.K[:n], k_new[None, :]])
        vals = np.vstack([self.V[:n], v_new[None, :]])
        alpha = attention_weights(q, keys, self.scale)
        out = attention_output(alpha, vals)
        if not self.evict:
            if n >= self.budget:
                raise ValueError("full-KV cache is at capacity")
            return StepResult(out, alpha, None, -1, n, False, [])
        if n < self.budget:
            return StepResult(out, alpha, None, -1, n, False, [])
        scores = longflow_scores(alpha[:, :n], self.vnorm[:n])
        scores[:self.sink_size] = np.inf
        victim = first_argmin(scores)
        tie, legal = near_tie_set(scores)
        return StepResult(out, alpha, scores, victim, victim, tie, legal)

    def _attend_deferred(self, q, k_new, v_new) -> StepResult:
        """The blog engine's order: write first (into the previous victim),
        then attend over the occupied slots, then pick the next victim."""
        n, B = self.n, self.budget
        if n < B:
            slot, replaced, n_after = n, -1, n + 1
        else:
            slot = self.victim if self.victim >= 0 else B - 1
            replaced, n_after = slot, n
        keys = self.K[:n_after].copy()
        vals = self.V[:n_after].copy()
        keys[slot] = k_new
        vals[slot] = v_new
        alpha = attention_weights(q, keys, self.scale)
        out = attention_output(alpha, vals)
        if n_after < B:
            return StepResult(out, alpha, None, replaced, slot, False, [])
        vnorm = self.vnorm[:n_after].copy()
        vnorm[slot] = value_norms(v_new[None, :], self.norm)[0]
        scores = longflow_scores(alpha, vnorm)
        scores[:self.sink_size] = np.inf
        scores[slot] = np.inf
        if not np.isfinite(scores).any():
            return StepResult(out, alpha, scores, replaced, slot, False, [-1], -1)
        nxt = first_argmin(scores)
        tie, legal = near_tie_set(scores)
        return StepResult(out, alpha, scores, replaced, slot, tie, legal, nxt)

    def commit(self, res: StepResult, k_new, v_new, slot: Optional[int] = None) -> None:
        """Write the new token. `slot` overrides the choice this step made (same
        order: the victim; deferred: the next victim), and must be legal."""
        if self.evict and self.order == "deferred":
            target = res.slot
            if res.evicted < 0:
                self.n += 1
            choice = res.next_victim if slot is None else int(slot)
            if choice != res.next_victim and choice not in res.legal:
                raise ValueError(f"slot {choice} is not a legal victim")
            self.victim = choice
        elif res.evicted < 0:
            target = res.slot
            self.n += 1
        else:
            target = res.evicted if slot is None else int(slot)
            if target not in res.legal and target != res.evicted:
                raise ValueError(f"slot {target} is not a legal eviction choice")
        self.K[target] = np.asarray(k_new, np.float64)
        self.V[target] = np.asarray(v_new, np.float64)
        self.vnorm[target] = value_norms(np.asarray(v_new, np.float64)[None, :], self.norm)[0]

    def step(self, q, k_new, v_new) -> StepResult:
        res = self.attend(q, k_new, v_new)
        self.commit(res, k_new, v_new)
        return res


class LayerCache:
    """All pairs of one layer: batch x num_kv_heads PairCache objects.

    Query head j uses KV head j // G (contiguous GQA groups).
    scope="kv_head": every pair chooses its own victim.
    scope="sequence": the KV heads of a sequence share one victim, the first
    argmin of the sum over heads (in head order) of their score vectors.
    """

    def __init__(self, batch: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, budget: int, sink_size: int = 0,
                 evict: bool = True, scale: Optional[float] = None,
                 pairs: Optional[list] = None, norm: str = "l1",
                 order: str = "same_step", scope: str = "kv_head"):
        if num_q_heads % num_kv_heads:
            raise ValueError("num_q_heads must be a multiple of num_kv_heads")
        if scope not in ("kv_head", "sequence"):
            raise ValueError("unknown scope")
        self.batch, self.hq, self.hkv = batch, num_q_heads, num_kv_heads
        self.group = num_q_heads // num_kv_heads
        self.head_dim = head_dim
        self.scope = scope
        self.order = order
        all_pairs = [(b, h) for b in range(batch) for h in range(num_kv_heads)]
        if pairs is not None and scope == "sequence":
            seqs = {b for b, _ in pairs}
            pairs = [(b, h) for b in sorted(seqs) for h in range(num_kv_heads)]
        self.pairs = all_pairs if pairs is None else [tuple(p) for p in pairs]
        self.cache = {p: PairCache(budget, head_dim, sink_size, evict, scale, norm, order)
                      for p in self.pairs}

    def prefill(self, k, v, n_per_seq) -> None:
        """k, v [batch][n_max][num_kv_heads][d]; sequence b keeps its first n_b
        rows; a negative n_b leaves sequence b as it is."""
        for (b, h), c in self.cache.items():
            n = int(n_per_seq[b])
            if n >= 0:
                c.prefill(k[b, :n, h], v[b, :n, h])

    def reset(self, seqs) -> None:
        """Recycle the regions of the given sequences (every KV head)."""
        for (b, h), c in self.cache.items():
            if b in seqs:
                c.reset()

    def attend(self, q, k_new, v_new):
        """q [batch][Hq][d], k_new/v_new [batch][Hkv][d] -> {pair: StepResult}."""
        g = self.group
        res = {(b, h): c.attend(q[b, h * g:(h + 1) * g], k_new[b, h], v_new[b, h])
               for (b, h), c in self.cache.items()}
        if self.scope == "sequence":
            self._share_victims(res)
        return res

    def _share_victims(self, res) -> None:
        """Replace each pair's own choice by its sequence's choice."""
        for b in sorted({b for b, _ in res}):
            heads = [res[(b, h)] for h in range(self.hkv)]
            if heads[0].scores is None:
                continue
            total = np.zeros_like(heads[0].scores)
            for r in heads:
                total = total + r.scores
            if not np.isfinite(total).any():
                choice, tie, legal = -1, False, [-1]
            else:
                choice = first_argmin(total)
                tie, legal = near_tie_set(total)
            for r in heads:
                r.scores_own = r.scores
                r.scores = total
                r.near_tie, r.legal = tie, legal
                if self.order == "deferred":
                    r.next_victim = choice
                else:
                    r.evicted = r.slot = choice

    def commit(self, results, k_new, v_new, slots=None) -> None:
        for (b, h), c in self.cache.items():
            s = None if slots is None else slots.get((b, h))
            c.commit(results[(b, h)], k_new[b, h], v_new[b, h], s)

    def step(self, q, k_new, v_new):
        res = self.attend(q, k_new, v_new)
        self.commit(res, k_new, v_new)
        return res

    def output(self, results) -> np.ndarray:
        """Assemble out [batch][Hq][d] for the pairs held (others are NaN)."""
        out = np.full((self.batch, self.hq, self.head_dim), np.nan)
        g = self.group
        for (b, h), r in results.items():
            out[b, h * g:(h + 1) * g] = r.out
        return out
